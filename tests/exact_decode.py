"""Inputs and expected outputs that make the layer's decoded trellis states
visible bit for bit through its output.

Row m of x is s_K * fp16(H[j] / sqrt(128)) on the 128-block of k_m = 128 b + j
and zero elsewhere, so the input rotation returns exactly the unit vector e_k:
every butterfly sum is an integer multiple of the fp16 value c = fp16(1/sqrt128)
(exact), and c * 128 / sqrt(128) = 0.99989... rounds to 1.0 in fp16. With
every column scale 1.0 and an integer codebook (state & 255, or state >> 8),
the GEMM output is then exactly cb[state(k_m, n)], the output rotation's
butterflies are exact integer sums S (|S| <= 128 * 255 < 2^24), and the only
rounding left is the kernels' fp32 product S * fp32(1/sqrt128) followed by one
fp16 rounding. The expected output below applies exactly that to the oracle's
states, so a single misdecoded state (which moves S by at least 1, and every
output of its 128-column block by about 0.088) changes the result.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg

import workloads as WL

H = scipy.linalg.hadamard(128).astype(np.int64)
C16 = np.float16(1.0 / np.sqrt(128.0))
INV_SQRT128_F32 = np.float32(1.0 / np.sqrt(128.0))
ONE16 = np.uint16(0x3C00)


def codebook(kind: str) -> np.ndarray:
    """65536 fp16 integers: the state's low byte ('lo') or high byte ('hi')."""
    s = np.arange(65536, dtype=np.int64)
    v = (s & 255) if kind == "lo" else (s >> 8)
    return v.astype(np.float16).view(np.uint16)


def unit_layer(seed: int, K: int, N: int, bits: int) -> dict:
    """A layer with random codes and signs and every column scale 1.0."""
    L = WL.layer(seed, K, N, 0, bits)
    return dict(L, scale=np.full(N, ONE16, np.uint16))


def unit_rows(ks, K: int, sign_k) -> np.ndarray:
    """Rows of x whose input rotation is exactly e_k for k in ks."""
    x = np.zeros((len(ks), K), np.float64)
    for m, k in enumerate(ks):
        b, j = divmod(int(k), 128)
        x[m, 128 * b:128 * b + 128] = H[j] * np.float64(C16)
    sk = np.where(np.asarray(sign_k, np.uint16) & 0x8000, -1.0, 1.0)
    return (x * sk).astype(np.float16).view(np.uint16)


def expected_y(states: np.ndarray, ks, kind: str, sign_n) -> np.ndarray:
    """The layer output for unit_rows(ks) under codebook(kind) and unit
    scales, from the states (K x N) and the kernels' fp32 scaling."""
    st = states[np.asarray(ks, np.int64)].astype(np.int64)
    v = (st & 255) if kind == "lo" else (st >> 8)
    M, N = v.shape
    S = (v.reshape(M, N // 128, 128) @ H.T).reshape(M, N)       # exact integers
    y = (S.astype(np.float32) * INV_SQRT128_F32).astype(np.float16).view(np.uint16)
    return y ^ (np.asarray(sign_n, np.uint16) & np.uint16(0x8000))
