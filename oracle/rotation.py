"""Incoherent processing for fp8 attention, oracle side.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The FlashAttention-3 snippets name "incoherent processing" beside block
quantisation as the way FA-3 lowers fp8 error, without defining it.  Reading
taken: Q and K are multiplied along the head dimension by the same random
orthogonal matrix M = diag(s) H_d / sqrt(d) before they are quantised, with
H_d the Sylvester-ordered Walsh-Hadamard matrix and s a vector of random
signs.  Because M M^T = I, (Q M)(K M)^T = Q K^T: the attention is unchanged,
while a large entry of a row is spread over all d coordinates before the
rounding to fp8.  V is not rotated.

Block quantisation is the one the fp8 path already uses: per (b, h) and
64-row block, scale = max|x| / 448 (1 for an all-zero block), value =
E4M3FN rounding of x / scale (nearest, ties to the even code).  The second
scale rule, used for V, takes the smallest power of two with
max|x| / scale <= 448 instead (the form of an E8M0 block scale).
"""
from __future__ import annotations

import numpy as np

from .codecs import round_to_e4m3fn

E4M3_MAX = 448.0


def hadamard_matrix(n: int) -> np.ndarray:
    """Sylvester's construction: H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]]."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    H = np.ones((1, 1))
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def incoherent_rotation(x, signs) -> np.ndarray:
    """x [..., d] -> x diag(signs) H_d / sqrt(d), in float64."""
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    d = x.shape[-1]
    return (x * s) @ hadamard_matrix(d) / np.sqrt(d)


def smallest_pow2_scale(amax: float) -> float:
    """The smallest power of two s with amax / s <= 448 (amax > 0): a first
    guess from log2, then moved until 448 * s >= amax > 448 * s / 2, both
    comparisons exact in float64."""
    k = int(np.ceil(np.log2(amax / E4M3_MAX)))
    while amax > E4M3_MAX * 2.0 ** k:
        k += 1
    while amax <= E4M3_MAX * 2.0 ** (k - 1):
        k -= 1
    return 2.0 ** k


def quantize_e4m3_blocks(x, block: int = 64, pow2: bool = False):
    """Block-quantise [..., N, d] rows: returns (dequantised values float64,
    scales float64 [..., ceil(N/block)], the pre-rounding ratios x / scale).
    The scale of a block is max|x| / 448, or with ``pow2`` the smallest power
    of two with max|x| / scale <= 448; 1 for an all-zero block."""
    x = np.asarray(x, dtype=np.float64)
    N = x.shape[-2]
    nb = -(-N // block)
    scales = np.empty(x.shape[:-2] + (nb,))
    ratio = np.empty_like(x)
    for i in range(nb):
        rows = slice(i * block, min((i + 1) * block, N))
        amax = np.max(np.abs(x[..., rows, :]), axis=(-2, -1))
        if pow2:
            s = np.vectorize(lambda a: smallest_pow2_scale(a) if a > 0 else 1.0,
                             otypes=[np.float64])(amax)
        else:
            s = np.where(amax > 0, amax / E4M3_MAX, 1.0)
        scales[..., i] = s
        ratio[..., rows, :] = x[..., rows, :] / s[..., None, None]
    vals = round_to_e4m3fn(ratio)
    rows = np.arange(N) // block
    return vals * scales[..., rows][..., None], scales, ratio
