"""Brute-force trellis decoder for tiny inputs (a test pin, not an oracle).

It follows the shift-register reading of the stand-in format rather than the
window formula the oracle uses: unpack every tile into its bit stream (256 *
bits bits), seed a 16-bit register with the first 16 bits, and for every step
emit the register and then shift in the next `bits` bits at the top. Because
the stream is tail-biting, the bits shifted in after the tile's last bit are
bits 0, 1, 2, ... again.
"""
import numpy as np


def tile_bits(words):
    bits = []
    for w in words:
        w = int(w)
        for b in range(32):
            bits.append((w >> b) & 1)
    return bits


def tile_states(words, bits_per_weight=4):
    b = bits_per_weight
    stream = tile_bits(words)
    assert len(stream) == 256 * b
    reg = 0
    for t in range(16):
        reg |= stream[t] << t
    states = []
    pos = 16
    for _ in range(256):
        states.append(reg)
        for t in range(b):
            reg = (reg >> 1) | (stream[pos % len(stream)] << 15)
            pos += 1
    return states


def states_matrix(codes, K, N, bits_per_weight=4):
    codes = np.asarray(codes, dtype=np.uint32)
    words_per_tile = 8 * bits_per_weight
    out = np.zeros((K, N), dtype=np.uint16)
    ntiles_n = N // 16
    for kt in range(K // 16):
        for nt in range(ntiles_n):
            t = kt * ntiles_n + nt
            st = tile_states(codes[t * words_per_tile:(t + 1) * words_per_tile], bits_per_weight)
            for step, s in enumerate(st):
                r, c = step % 16, step // 16
                out[kt * 16 + r, nt * 16 + c] = s
    return out
