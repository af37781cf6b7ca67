"""Brute-force trellis decoder for tiny inputs (a test pin, not an oracle).

It follows the shift-register reading of the stand-in format rather than the
window formula the oracle uses: unpack every tile into its 1024-bit stream, seed
a 16-bit register with the first 16 bits, and for every step emit the register
and then shift in the next 4 bits at the top. Because the stream is tail-biting,
the bits shifted in after bit 1023 are bits 0, 1, 2, ... again.
"""
import numpy as np


def tile_bits(words):
    bits = []
    for w in words:
        w = int(w)
        for b in range(32):
            bits.append((w >> b) & 1)
    return bits


def tile_states(words):
    bits = tile_bits(words)
    assert len(bits) == 1024
    reg = 0
    for t in range(16):
        reg |= bits[t] << t
    states = []
    pos = 16
    for _ in range(256):
        states.append(reg)
        nib = 0
        for t in range(4):
            nib |= bits[pos % 1024] << t
            pos += 1
        reg = (reg >> 4) | (nib << 12)
    return states


def states_matrix(codes, K, N):
    codes = np.asarray(codes, dtype=np.uint32)
    out = np.zeros((K, N), dtype=np.uint16)
    ntiles_n = N // 16
    for kt in range(K // 16):
        for nt in range(ntiles_n):
            t = kt * ntiles_n + nt
            st = tile_states(codes[t * 32:(t + 1) * 32])
            for step, s in enumerate(st):
                r, c = step % 16, step // 16
                out[kt * 16 + r, nt * 16 + c] = s
    return out
