"""Decoders from stored bit patterns to exact float64 values (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The GPU kernels read the same bits; the oracle evaluates attention on the
exact real values those bits stand for, so that the only differences left are
the kernel's own rounding.
"""
from __future__ import annotations

import numpy as np


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.

    bfloat16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent
    bits (bias 127), 7 fraction bits.  Normal: (-1)^s * 2^(E-127) * (1+F/128);
    subnormal (E=0): (-1)^s * 2^-126 * F/128; E=255: inf (F=0) or NaN.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = (b >> 15) & 1
    E = (b >> 7) & 0xFF
    F = b & 0x7F
    sign = np.where(s == 1, -1.0, 1.0)
    normal = sign * np.ldexp(1.0 + F / 128.0, (E - 127).astype(np.int32))
    sub = sign * np.ldexp(F / 128.0, -126)
    out = np.where(E == 0, sub, normal)
    out = np.where((E == 255) & (F == 0), sign * np.inf, out)
    out = np.where((E == 255) & (F != 0), np.nan, out)
    return out


def decode_f16(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64.

    1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.  Normal:
    (-1)^s * 2^(E-15) * (1+F/1024); subnormal (E=0): (-1)^s * 2^-14 * F/1024;
    E=31: inf (F=0) or NaN.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = (b >> 15) & 1
    E = (b >> 10) & 0x1F
    F = b & 0x3FF
    sign = np.where(s == 1, -1.0, 1.0)
    normal = sign * np.ldexp(1.0 + F / 1024.0, (E - 15).astype(np.int32))
    sub = sign * np.ldexp(F / 1024.0, -14)
    out = np.where(E == 0, sub, normal)
    out = np.where((E == 31) & (F == 0), sign * np.inf, out)
    out = np.where((E == 31) & (F != 0), np.nan, out)
    return out


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN codes (uint8) -> float64.

    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Normal (E>=1):
    (-1)^s * 2^(E-7) * (1+M/8); subnormal (E=0): (-1)^s * 2^-6 * M/8.
    There are no infinities; S.1111.111 (0x7F / 0xFF) is NaN, so the largest
    finite magnitude is 0x7E = 2^8 * 1.75 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    E = (c >> 3) & 0xF
    M = c & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    normal = sign * np.ldexp(1.0 + M / 8.0, (E - 7).astype(np.int32))
    sub = sign * np.ldexp(M / 8.0, -6)
    out = np.where(E == 0, sub, normal)
    out = np.where((E == 15) & (M == 7), np.nan, out)
    return out


def dequant_fp8_rows(codes: np.ndarray, scales: np.ndarray, block: int = 64) -> np.ndarray:
    """Block-scaled fp8 -> float64: x_hat[..., n, c] = value(code) * scale[..., n // block].

    ``codes`` is [..., N, d]; ``scales`` is [..., ceil(N/block)] float32.
    """
    vals = decode_e4m3fn(codes)
    N = vals.shape[-2]
    rows = np.arange(N) // block
    s = np.asarray(scales, dtype=np.float64)[..., rows]
    return vals * s[..., :, None]


def round_to_e4m3fn(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest E4M3FN value, ties to the even code,
    saturating at +-448; returns float64 values (not codes).

    Written as a search over the decoded grid of the 127 non-negative finite
    codes (0x00..0x7E, whose values increase with the code), so it depends on
    nothing but ``decode_e4m3fn``.
    """
    grid = decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))      # 0 .. 448, increasing
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), grid[-1])
    hi = np.clip(np.searchsorted(grid, a, side="left"), 1, len(grid) - 1)
    lo = hi - 1
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    r = np.where(pick_hi, grid[hi], grid[lo])
    return np.where(np.signbit(x), -r, r)
