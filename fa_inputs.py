"""Seeded synthetic inputs for the attention kernels and for the CPU oracle.

This module is shared by the GPU path's tests/bench and by the oracle's tests.
It only *makes* inputs; it holds none of the attention arithmetic.  What it
does:

* draws i.i.d. N(0,1) float32 values from one numpy PCG64 stream per
  (workload, tensor, batch, head), so any (b, h) slice can be regenerated on
  its own without materialising the whole tensor;
* rounds float32 to bfloat16 or IEEE fp16 bit patterns (round to nearest,
  ties to even);
* for the fp8 workload, injects x20 outliers with probability 1e-3 per element
  (each tensor has its own mask stream) and quantises to OCP FP8 E4M3FN codes
  with one float32 scale per 64 consecutive sequence rows of each (b, h),
  ``scale = amax / 448`` for Q and K, the smallest power of two with
  ``amax / scale <= 448`` for V, and
  ``code = round_to_nearest_even_saturating(x / scale)``.

Workload shapes follow the configurations the kernels are measured on (see
``WORKLOADS``).  Attention is defined per (batch, head) on ``[B, H, N, d]``
row-major tensors, the layout the pages use for Q, K, V and O (FlashAttention
note, "问题分析": ``(batch, heads, seq_len, head_dim)``).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED_ROOT = 20261202
Q_ID, K_ID, V_ID = 0, 1, 2
OUTLIER_MASK_ID = {Q_ID: 3, K_ID: 4, V_ID: 5}
DO_ID = 6          # the upstream gradient dO of a backward pass
SIGNS_ID = 7       # the random signs of an incoherent rotation
FP8_BLOCK_ROWS = 64
# V's block scales are powers of two (the E8M0 form of the matrix cores'
# operand scale); Q's and K's are amax / 448, which keeps a block's largest
# element exact
FP8_POW2_SCALE = {Q_ID: False, K_ID: False, V_ID: True}
E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    """One measured configuration.  ``kind`` is 'fwd', 'fwd_fp8', 'decode' or
    'decode_gqa' (``H`` query heads over ``Hkv`` key/value heads)."""
    wid: int
    name: str
    kind: str
    B: int
    H: int
    N: int          # query length (== key length for prefill); 1 for decode
    d: int
    Lkv: int = 0    # decode only: KV-cache length
    num_splits: int = 0
    causal: tuple = (False,)
    out_dtype: str = "bf16"
    Hkv: int = 0    # decode_gqa only: key/value heads
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


WORKLOADS = {
    1: Workload(1, "single_head_b1h1n128d64", "fwd", 1, 1, 128, 64,
                causal=(False,), out_dtype="fp32",
                note="B=1 H=1 N=128 d=64, non-causal, fp32 output"),
    2: Workload(2, "llama7b_layer_b2h32n2048d128", "fwd", 2, 32, 2048, 128,
                causal=(False, True), out_dtype="bf16",
                note="LLaMA-7B-shaped layer, causal and non-causal"),
    3: Workload(3, "long_causal_b1h16n16384d128", "fwd", 1, 16, 16384, 128,
                causal=(True,), out_dtype="bf16",
                note="single batch, 16 heads, N=16384, causal"),
    4: Workload(4, "decode_b8h32lkv65536d128s64", "decode", 8, 32, 1, 128,
                Lkv=65536, num_splits=64, causal=(False,), out_dtype="bf16",
                note="one query per (b,h), 64 KiB-key cache, 64 splits"),
    5: Workload(5, "fp8_causal_b4h16n8192d128", "fwd_fp8", 4, 16, 8192, 128,
                causal=(True,), out_dtype="bf16",
                note="e4m3 Q/K/V, one fp32 scale per 64 rows per head (V's powers of two), "
                     "0.1% x20 outliers"),
    6: Workload(6, "decode_gqa_b8hq64hkv8lkv65536d128s64", "decode_gqa", 8, 64, 1, 128,
                Lkv=65536, num_splits=64, Hkv=8, causal=(False,), out_dtype="bf16",
                note="grouped K/V heads (8 query heads per K/V head), 64 KiB-key cache"),
    7: Workload(7, "decode_mqa_b8hq32hkv1lkv65536d128s64", "decode_gqa", 8, 32, 1, 128,
                Lkv=65536, num_splits=64, Hkv=1, causal=(False,), out_dtype="bf16",
                note="one shared K/V head for 32 query heads, 64 KiB-key cache"),
}


# A ragged chunked-prefill batch: 8 sequences, each a chunk of new queries
# (lq) against its cached keys plus itself (lk = cached + lq), H=32, d=128,
# causal masking aligned at the sequence end.  Lengths mix short and long
# chunks and short and long caches.
VARLEN_PREFILL = {
    "wid": 8, "name": "chunked_prefill_ragged_b8h32d128", "H": 32, "d": 128,
    "lq": [2048, 1024, 512, 256, 1536, 768, 128, 1800],
    "lk": [2048, 2048, 4608, 6256, 2048, 2816, 8192, 2048],
}


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------------------
# random streams
# ---------------------------------------------------------------------------

def stream(wid: int, tensor_id: int, b: int, h: int) -> np.random.Generator:
    """The PCG64 stream of one (workload, tensor, batch, head)."""
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([SEED_ROOT, wid, tensor_id, b, h])))


def normals(wid: int, tensor_id: int, b: int, h: int, rows: int, d: int) -> np.ndarray:
    """float32 [rows, d] i.i.d. N(0,1) for one (b, h)."""
    return stream(wid, tensor_id, b, h).standard_normal(size=(rows, d), dtype=np.float32)


# ---------------------------------------------------------------------------
# float32 -> bfloat16 bits (round to nearest, ties to even)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even; uint16 bits.

    NaN stays a quiet NaN; values that round past the largest finite bf16
    become infinity, as IEEE rounding does.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest IEEE binary16, ties to even
    (numpy's float32 -> float16 conversion); uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------------------
# float -> OCP FP8 E4M3FN codes (bias 7, no infinities, 0x7F/0xFF are NaN)
# ---------------------------------------------------------------------------

def f64_to_e4m3fn_codes(y: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3FN value, ties to even, saturating at +-448.

    The E4M3FN grid: exponent field 1..15 gives normals 2^(e-7)*(1+m/8);
    exponent field 0 gives subnormals m*2^-9; the largest finite value is
    0x7E = 1.75*2^8 = 448 (0x7F is NaN).  Inputs are finite.
    """
    y = np.asarray(y, dtype=np.float64)
    sign = np.signbit(y)
    a = np.abs(y)
    # binade exponent e with 2^e <= a < 2^(e+1); below the normal range the
    # quantum stays that of the subnormals (2^-9)
    _, ex = np.frexp(a)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    quantum = np.ldexp(1.0, (e - 3).astype(np.int32))
    mag = np.rint(a / quantum) * quantum          # np.rint rounds half to even
    mag = np.minimum(mag, E4M3_MAX)
    # encode the (now representable) magnitude
    codes = np.zeros(a.shape, dtype=np.uint8)
    sub = mag < 2.0 ** -6
    codes[sub] = np.rint(mag[sub] / 2.0 ** -9).astype(np.uint8)
    nm = ~sub
    if nm.any():
        f, ex2 = np.frexp(mag[nm])                  # mag = f*2^ex2, f in [0.5,1)
        E = ex2.astype(np.int64) - 1
        mant = np.rint((f * 2.0 - 1.0) * 8.0).astype(np.int64)
        codes[nm] = ((E + 7) << 3 | mant).astype(np.uint8)
    codes[sign & (codes != 0)] |= np.uint8(0x80)
    return codes


def pow2_scale(amax: float) -> float:
    """The smallest power of two s with amax / s <= 448, from the binary
    exponent: amax = f * 2^e with f in [0.5, 1) and 448 = 0.875 * 2^9, so
    s = 2^(e - 9) when f <= 0.875, else 2^(e - 8)."""
    f, e = np.frexp(np.float64(amax))
    return float(np.ldexp(1.0, int(e) - 9 if f <= 0.875 else int(e) - 8))


def quantize_e4m3_rows(x: np.ndarray, block: int = FP8_BLOCK_ROWS, pow2: bool = False):
    """Quantise one (b, h) slice ``x`` float32 [N, d] with per-``block``-row scales.

    Returns (codes uint8 [N, d], scales float32 [ceil(N/block)]).
    ``scale = amax/448`` in float32, or with ``pow2`` the smallest power of
    two with amax / scale <= 448 (1.0 for an all-zero block either way); each
    element is encoded from ``x / scale`` evaluated in float64.
    """
    N, d = x.shape
    nb = (N + block - 1) // block
    codes = np.empty((N, d), dtype=np.uint8)
    scales = np.empty(nb, dtype=np.float32)
    for i in range(nb):
        blk = x[i * block:(i + 1) * block]
        amax = np.float32(np.max(np.abs(blk))) if blk.size else np.float32(0)
        if amax == 0:
            s = np.float32(1.0)
        elif pow2:
            s = np.float32(pow2_scale(amax))
        else:
            s = np.float32(amax / np.float32(E4M3_MAX))
        scales[i] = s
        codes[i * block:(i + 1) * block] = f64_to_e4m3fn_codes(
            blk.astype(np.float64) / np.float64(s))
    return codes, scales


# ---------------------------------------------------------------------------
# whole tensors and single slices
# ---------------------------------------------------------------------------

def bf16_slice(wid: int, tensor_id: int, b: int, h: int, rows: int, d: int) -> np.ndarray:
    return f32_to_bf16_bits(normals(wid, tensor_id, b, h, rows, d))


def bf16_tensor(wid: int, tensor_id: int, B: int, H: int, rows: int, d: int,
                out: np.ndarray | None = None) -> np.ndarray:
    """uint16 [B, H, rows, d] bf16 bits, generated per (b, h) in parallel."""
    if out is None:
        out = np.empty((B, H, rows, d), dtype=np.uint16)

    def fill(bh):
        b, h = divmod(bh, H)
        out[b, h] = bf16_slice(wid, tensor_id, b, h, rows, d)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(B * H)))
    return out


def f16_tensor(wid: int, tensor_id: int, B: int, H: int, rows: int, d: int) -> np.ndarray:
    """uint16 [B, H, rows, d] IEEE fp16 bits of the same normals as bf16_tensor."""
    out = np.empty((B, H, rows, d), dtype=np.uint16)

    def fill(bh):
        b, h = divmod(bh, H)
        out[b, h] = f32_to_f16_bits(normals(wid, tensor_id, b, h, rows, d))

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(B * H)))
    return out


def fp8_slice(wid: int, tensor_id: int, b: int, h: int, rows: int, d: int,
              outlier_p: float = 1e-3, outlier_mult: float = 20.0, pow2: bool | None = None):
    """One (b, h) of an fp8 workload tensor: (codes [rows, d], scales [ceil(rows/64)]).
    ``pow2`` None takes the tensor's rule from FP8_POW2_SCALE."""
    x = normals(wid, tensor_id, b, h, rows, d)
    if outlier_p > 0:
        m = stream(wid, OUTLIER_MASK_ID[tensor_id], b, h).random(size=(rows, d)) < outlier_p
        x[m] *= np.float32(outlier_mult)
    return quantize_e4m3_rows(x, pow2=FP8_POW2_SCALE[tensor_id] if pow2 is None else pow2)


def outlier_bf16_tensor(wid: int, tensor_id: int, B: int, H: int, rows: int, d: int,
                        outlier_p: float = 1e-3, outlier_mult: float = 20.0) -> np.ndarray:
    """uint16 bf16 bits [B, H, rows, d]: the fp8 workload's values (N(0,1) with
    x20 outliers at rate 1e-3, same streams) rounded to bf16 instead of being
    quantised, as the input of an on-GPU quantisation."""
    out = np.empty((B, H, rows, d), dtype=np.uint16)

    def fill(bh):
        b, h = divmod(bh, H)
        x = normals(wid, tensor_id, b, h, rows, d)
        if outlier_p > 0:
            m = stream(wid, OUTLIER_MASK_ID[tensor_id], b, h).random(size=(rows, d)) < outlier_p
            x[m] *= np.float32(outlier_mult)
        out[b, h] = f32_to_bf16_bits(x)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(B * H)))
    return out


def rotation_signs(wid: int, d: int) -> np.ndarray:
    """float32 [d] of +-1: the random signs of an incoherent rotation."""
    return stream(wid, SIGNS_ID, 0, 0).choice(np.array([-1.0, 1.0], np.float32), size=d)


def fp8_tensor(wid: int, tensor_id: int, B: int, H: int, rows: int, d: int,
               outlier_p: float = 1e-3, outlier_mult: float = 20.0, pow2: bool | None = None):
    """(codes uint8 [B,H,rows,d], scales float32 [B,H,ceil(rows/64)])."""
    nb = (rows + FP8_BLOCK_ROWS - 1) // FP8_BLOCK_ROWS
    codes = np.empty((B, H, rows, d), dtype=np.uint8)
    scales = np.empty((B, H, nb), dtype=np.float32)

    def fill(bh):
        b, h = divmod(bh, H)
        codes[b, h], scales[b, h] = fp8_slice(wid, tensor_id, b, h, rows, d,
                                              outlier_p, outlier_mult, pow2)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(B * H)))
    return codes, scales


def workload_inputs(w: Workload):
    """All inputs of a workload as numpy arrays (bits, not values).

    fwd:     dict(q, k, v) uint16 bf16 bits [B,H,N,d]
    fwd_fp8: dict(q, k, v) uint8 e4m3 codes + (q_scale, k_scale, v_scale) float32
    decode:  dict(q [B,H,1,d], k [B,H,Lkv,d], v [B,H,Lkv,d]) uint16 bf16 bits
    decode_gqa: the same with k, v [B,Hkv,Lkv,d]
    """
    if w.kind == "fwd":
        return {n: bf16_tensor(w.wid, t, w.B, w.H, w.N, w.d)
                for n, t in (("q", Q_ID), ("k", K_ID), ("v", V_ID))}
    if w.kind == "fwd_fp8":
        r = {}
        for n, t in (("q", Q_ID), ("k", K_ID), ("v", V_ID)):
            r[n], r[n + "_scale"] = fp8_tensor(w.wid, t, w.B, w.H, w.N, w.d)
        return r
    if w.kind == "decode":
        return {"q": bf16_tensor(w.wid, Q_ID, w.B, w.H, 1, w.d),
                "k": bf16_tensor(w.wid, K_ID, w.B, w.H, w.Lkv, w.d),
                "v": bf16_tensor(w.wid, V_ID, w.B, w.H, w.Lkv, w.d)}
    if w.kind == "decode_gqa":
        return {"q": bf16_tensor(w.wid, Q_ID, w.B, w.H, 1, w.d),
                "k": bf16_tensor(w.wid, K_ID, w.B, w.Hkv, w.Lkv, w.d),
                "v": bf16_tensor(w.wid, V_ID, w.B, w.Hkv, w.Lkv, w.d)}
    raise ValueError(w.kind)
