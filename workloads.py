"""Seeded synthetic inputs for the EXL3-style trellis-quantized linear layer.

This module only draws random numbers and casts them to storage types. It holds
none of the method's arithmetic: no trellis decode, no Hadamard, no product.
Both the CPU oracle (via the tests) and the HIP path (via the tests and the
benchmark) receive the arrays it returns, so the two sides never generate their
own inputs.

Shapes and distributions follow the workloads the pages measure on:
  * MLP geometries K5120 x N17408 and K17408 x N5120 and the 32768-column wide
    projection (vLLM PR #316, follow-up item 2, the hgemm vs torch.mm table);
  * activations drawn as 0.05 * randn, the priming distribution of vLLM PR #314
    and PR #316 follow-up item 5;
  * the padded-logits widths 248077 / 248192 / 248320 (pegainfer PR #1046,
    Testing section).
The trellis format itself is not defined on the pages; the synthetic stand-in
(4 bits per weight, 16x16 tiles, 16-bit tail-biting bitshift state, LSB-first
32-bit words, a 65536-entry fp16 N(0,1) codebook, per-column fp16 scales and
+-1 sign vectors) is specified in include/exl3.h.

Every tensor comes from its own numpy PCG64 stream seeded with
[config_seed, tensor_id, *extra]; see `rng`.
"""
from __future__ import annotations

import numpy as np

# Codebook seed, shared by every configuration.
CB_SEED = 1000

# Per-configuration seeds.
SEED_TINY = 1
SEED_DECODE = 2
SEED_PREFILL = 3
SEED_WIDE = 4
SEED_LOGITS = 5

# Tensor ids inside a configuration's seed space.
T_CODES, T_SCALE, T_SIGN_K, T_SIGN_N, T_X, T_LOGITS_W = 0, 1, 2, 3, 4, 5

LOGITS_CHUNK_ROWS = 8192

FP16_ONE = np.uint16(0x3C00)
FP16_MINUS_ONE = np.uint16(0xBC00)


def rng(config_seed: int, tensor_id: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([int(config_seed), int(tensor_id), *[int(e) for e in extra]])


def codebook() -> np.ndarray:
    """65536 fp16 codebook entries (as uint16 bit patterns), N(0,1) rounded to fp16."""
    return np.random.default_rng(CB_SEED).standard_normal(65536).astype(np.float16).view(np.uint16)


def signs(config_seed: int, tensor_id: int, n: int, *extra: int) -> np.ndarray:
    bits = rng(config_seed, tensor_id, *extra).integers(0, 2, size=n, dtype=np.int64)
    return np.where(bits == 1, FP16_ONE, FP16_MINUS_ONE).astype(np.uint16)


def layer(config_seed: int, K: int, N: int, set_id: int = 0, bits: int = 4) -> dict:
    """One quantized layer: packed codes (uint32 words), column scales, sign vectors.

    codes has K*N*bits/32 uint32 words (bits per weight, 1..8; the 4-bit codes
    come from the stream of [config_seed, T_CODES, set_id], other widths from
    [config_seed, T_CODES, set_id, bits]); scale, sign_k and sign_n are fp16 bit
    patterns (uint16).
    """
    if K % 128 or N % 128:
        raise ValueError("K and N must be multiples of 128")
    if not 1 <= bits <= 8:
        raise ValueError("bits must be in 1..8")
    stream = rng(config_seed, T_CODES, set_id) if bits == 4 else rng(config_seed, T_CODES, set_id, bits)
    codes = stream.integers(0, 2**32, size=K * N * bits // 32, dtype=np.uint32)
    scale = rng(config_seed, T_SCALE, set_id).uniform(0.005, 0.02, size=N)
    scale = scale.astype(np.float16).view(np.uint16)
    return {
        "K": K,
        "N": N,
        "bits": bits,
        "codes": codes,
        "scale": scale,
        "sign_k": signs(config_seed, T_SIGN_K, K, set_id),
        "sign_n": signs(config_seed, T_SIGN_N, N, set_id),
    }


def activations(config_seed: int, M: int, K: int, *extra: int) -> np.ndarray:
    """M x K fp16 activations drawn as 0.05 * N(0,1), as uint16 bit patterns."""
    x = 0.05 * rng(config_seed, T_X, M, *extra).standard_normal((M, K))
    return x.astype(np.float16).view(np.uint16)


def logits_weights(config_seed: int, w_rows: int, K: int, threads: int = 8) -> np.ndarray:
    """w_rows x K fp16 output-projection rows drawn as 0.02 * N(0,1) (float32
    draws), in 8192-row chunks, each chunk from its own stream."""
    from concurrent.futures import ThreadPoolExecutor

    out = np.empty((w_rows, K), dtype=np.uint16)

    def fill(c):
        r0 = c * LOGITS_CHUNK_ROWS
        r1 = min(w_rows, r0 + LOGITS_CHUNK_ROWS)
        block = rng(config_seed, T_LOGITS_W, c).standard_normal((r1 - r0, K), dtype=np.float32)
        out[r0:r1] = (np.float32(0.02) * block).astype(np.float16).view(np.uint16)

    n_chunks = (w_rows + LOGITS_CHUNK_ROWS - 1) // LOGITS_CHUNK_ROWS
    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, range(n_chunks)))
    return out


# The five workload configurations, by what they are and their sizes.
TINY = {"name": "tiny K256xN256", "seed": SEED_TINY, "K": 256, "N": 256, "M": (1, 16, 128)}
DECODE = {"name": "decode K5120xN17408", "seed": SEED_DECODE, "K": 5120, "N": 17408,
          "M": (1, 4, 8, 16), "weight_sets": 12}
PREFILL = {"name": "prefill MLP", "seed": SEED_PREFILL,
           "geometries": ((5120, 17408), (17408, 5120)), "M": (128, 256, 1024, 2048, 4096),
           "weight_sets": 6}
WIDE = {"name": "wide K5120xN32768", "seed": SEED_WIDE, "K": 5120, "N": 32768, "M": (2048,)}
LOGITS = {"name": "padded logits K5120", "seed": SEED_LOGITS, "K": 5120, "n_valid": 248077,
          "w_rows": 248320, "M": (1, 16)}
