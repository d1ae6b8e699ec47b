"""The Python binding refuses tensors too small for the shapes a call states.

The C entry points take plain pointers and cannot see buffer sizes, so a
short tensor would let a kernel read or write past its end.  The binding
checks every tensor argument against the dense layout of include/fa.h before
it calls the library.  These tests use stand-in tensor objects: the checks
raise before any library call, so nothing touches a device.
"""
import pytest

import exact_attention_116_amd as fa


class Fake:
    """Just enough of a device tensor for the binding's checks.  The dtype
    defaults to the usual one of its element size (bf16, fp32, uint8)."""

    DEFAULT = {1: "torch.uint8", 2: "torch.bfloat16", 4: "torch.float32"}

    def __init__(self, numel, elem=2, dtype=None):
        self._n, self._e = numel, elem
        self.dtype = dtype or self.DEFAULT[elem]
        self.is_cuda = True

    def is_contiguous(self):
        return True

    def numel(self):
        return self._n

    def element_size(self):
        return self._e

    def data_ptr(self):
        return 0x1000


def raises_short(name, fn, *args, **kw):
    with pytest.raises(fa.FaError) as e:
        fn(*args, **kw)
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    assert str(e.value).startswith(f"{name} holds"), str(e.value)


def test_ptr_accepts_exact_size_and_rejects_one_byte_less():
    assert fa._ptr(Fake(8, 2), 16, "x") == 0x1000
    with pytest.raises(fa.FaError):
        fa._ptr(Fake(8, 2), 17, "x")
    assert fa._ptr(None, 100) is None
    assert fa._ptr(1234, 10 ** 9) == 1234          # raw addresses are the caller's


def test_dims_product():
    assert fa._n(2, 3, 4) == 24
    assert fa._n(2, -1, 4) == 0                     # negative: left to the library


def test_forward_sizes():
    B, H, N, d = 2, 3, 100, 64
    full, rows = B * H * N * d, B * H * N
    ok = lambda: Fake(full)
    raises_short("q", fa.fa_fwd, Fake(full - 1), ok(), ok(), ok(), Fake(rows, 4), B, H, N, d, 0.1, True)
    raises_short("v", fa.fa_fwd, ok(), ok(), Fake(full - 1), ok(), Fake(rows, 4), B, H, N, d, 0.1, True)
    raises_short("lse", fa.fa_fwd, ok(), ok(), ok(), ok(), Fake(rows - 1, 4), B, H, N, d, 0.1, True)
    # fp32 output needs four bytes per element
    raises_short("o", fa.fa_fwd_ex, ok(), ok(), ok(), Fake(full, 2), Fake(rows, 4), B, H, N, d, 0.1,
                 False, out_dtype=fa.FA_FP32)
    # fp8 inputs are one byte per element, with one fp32 scale per 64 rows
    nsb = B * H * ((N + 63) // 64)
    fp8 = lambda: Fake(full, 1)
    raises_short("k_scale", fa.fa_fwd_ex, fp8(), fp8(), fp8(), ok(), Fake(rows, 4), B, H, N, d, 0.1,
                 True, in_dtype=fa.FA_FP8_E4M3, q_scale=Fake(nsb, 4), k_scale=Fake(nsb - 1, 4),
                 v_scale=Fake(nsb, 4))


def test_decode_sizes():
    B, Hq, Hkv, L, d = 2, 8, 2, 300, 128
    q = lambda: Fake(B * Hq * d)
    c = lambda: Fake(B * Hkv * L * d)
    raises_short("kcache", fa.fa_decode_splitkv_gqa, q(), Fake(B * Hkv * L * d - 1), c(), q(),
                 None, B, Hq, Hkv, L, d, 4, 0.1)
    raises_short("lse", fa.fa_decode_splitkv_gqa, q(), c(), c(), q(), Fake(B * Hq - 1, 4),
                 B, Hq, Hkv, L, d, 4, 0.1)
    raises_short("workspace", fa.fa_decode_splitkv_gqa, q(), c(), c(), q(), None, B, Hq, Hkv, L, d,
                 4, 0.1, workspace=Fake(100, 1), workspace_bytes=101)
    raises_short("seqlens_k", fa.fa_decode_splitkv_varlen, q(), c(), c(), q(), None,
                 Fake(B - 1, 4, "torch.int32"), B, Hq, Hkv, L, d, 4, 0.1)
    H = 4
    raises_short("vcache", fa.fa_decode_splitkv, Fake(B * H * d), Fake(B * H * L * d),
                 Fake(B * H * L * d - 1), Fake(B * H * d), B, H, L, d, 8)


def test_varlen_and_quantize_and_backward_sizes():
    B, H, d, tq, tk = 3, 2, 64, 50, 70
    cu = lambda n: Fake(n, 4, "torch.int32")
    raises_short("cu_seqlens_k", fa.fa_fwd_varlen, Fake(tq * H * d), Fake(tk * H * d),
                 Fake(tk * H * d), Fake(tq * H * d), Fake(H * tq, 4), cu(B + 1), cu(B),
                 B, H, 30, 40, tq, tk, d, 0.1, True)
    raises_short("k", fa.fa_fwd_varlen, Fake(tq * H * d), Fake(tq * H * d), Fake(tk * H * d),
                 Fake(tq * H * d), Fake(H * tq, 4), cu(B + 1), cu(B + 1),
                 B, H, 30, 40, tq, tk, d, 0.1, True)
    N = 130
    raises_short("scales", fa.fa_fp8_quantize, Fake(B * H * N * d), Fake(d, 4), Fake(B * H * N * d, 1),
                 Fake(B * H * 2, 4), B, H, N, d)
    raises_short("signs", fa.fa_fp8_quantize, Fake(B * H * N * d), Fake(d - 1, 4),
                 Fake(B * H * N * d, 1), Fake(B * H * 3, 4), B, H, N, d)
    # the scale-rule form checks the same buffers
    raises_short("scales", fa.fa_fp8_quantize, Fake(B * H * N * d), None, Fake(B * H * N * d, 1),
                 Fake(B * H * 2, 4), B, H, N, d, scale_rule=fa.FA_FP8_SCALE_POW2)
    raises_short("codes", fa.fa_fp8_quantize, Fake(B * H * N * d), None, Fake(B * H * N * d - 1, 1),
                 Fake(B * H * 3, 4), B, H, N, d, scale_rule=fa.FA_FP8_SCALE_POW2)
    t = lambda: Fake(B * H * N * d)
    raises_short("dk", fa.fa_bwd, t(), t(), t(), t(), t(), Fake(B * H * N, 4), t(),
                 Fake(B * H * N * d - 1), t(), B, H, N, d, 0.1, True)
    h = lambda: Fake(B * H * N * d, 2, "torch.float16")
    raises_short("dout", fa.fa_bwd_ex, h(), h(), h(), h(), Fake(10, 2, "torch.float16"),
                 Fake(B * H * N, 4), h(), h(), h(), B, H, N, d, 0.1, True, dtype=fa.FA_FP16)
    # packed backward: q-side tensors hold total_q rows, k-side total_k, lse H * total_q
    qs, ks = (lambda: Fake(tq * H * d)), (lambda: Fake(tk * H * d))
    raises_short("dv", fa.fa_bwd_varlen, qs(), ks(), ks(), qs(), qs(), Fake(H * tq, 4), qs(), ks(),
                 Fake(tk * H * d - 1), cu(B + 1), cu(B + 1), B, H, 30, 40, tq, tk, d, 0.1, True)
    raises_short("lse", fa.fa_bwd_varlen, qs(), ks(), ks(), qs(), qs(), Fake(H * tq - 1, 4), qs(),
                 ks(), ks(), cu(B + 1), cu(B + 1), B, H, 30, 40, tq, tk, d, 0.1, True)
    raises_short("cu_seqlens_q", fa.fa_bwd_varlen, qs(), ks(), ks(), qs(), qs(), Fake(H * tq, 4),
                 qs(), ks(), ks(), cu(B), cu(B + 1), B, H, 30, 40, tq, tk, d, 0.1, True)


def raises_dtype(name, fn, *args, **kw):
    with pytest.raises(fa.FaError) as e:
        fn(*args, **kw)
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    assert str(e.value).startswith(f"{name} has dtype"), str(e.value)


def test_dtypes_are_checked():
    """A tensor of another element type but enough bytes is refused: its bits
    would otherwise be read as the stated type."""
    B, H, N, d = 1, 2, 64, 64
    full, rows = B * H * N * d, B * H * N
    ok = lambda: Fake(full)
    f32 = lambda n: Fake(n, 4)
    # a float32 q (twice the bytes) and a bf16 lse (enough bytes at double count)
    raises_dtype("q", fa.fa_fwd, f32(full), ok(), ok(), ok(), f32(rows), B, H, N, d, 0.1, True)
    raises_dtype("lse", fa.fa_fwd, ok(), ok(), ok(), ok(), Fake(2 * rows, 2), B, H, N, d, 0.1, True)
    # fp16 inputs with a bf16 v; fp32 output asked for with a bf16 o
    h = lambda: Fake(full, 2, "torch.float16")
    raises_dtype("v", fa.fa_fwd_ex, h(), h(), ok(), h(), f32(rows), B, H, N, d, 0.1, True,
                 in_dtype=fa.FA_FP16, out_dtype=fa.FA_FP16)
    raises_dtype("o", fa.fa_fwd_ex, ok(), ok(), ok(), Fake(2 * full, 2), f32(rows), B, H, N, d, 0.1,
                 True, out_dtype=fa.FA_FP32)
    # fp8 codes may be uint8, int8 or float8_e4m3fn; scales must be fp32
    nsb = B * H * ((N + 63) // 64)
    for codes_dt in ("torch.uint8", "torch.int8", "torch.float8_e4m3fn"):
        c = lambda: Fake(full, 1, codes_dt)
        raises_dtype("v_scale", fa.fa_fwd_ex, c(), c(), c(), ok(), f32(rows), B, H, N, d, 0.1, True,
                     in_dtype=fa.FA_FP8_E4M3, q_scale=f32(nsb), k_scale=f32(nsb),
                     v_scale=Fake(2 * nsb, 2))
    # int32 lengths for the packed and per-sequence calls
    raises_dtype("cu_seqlens_q", fa.fa_fwd_varlen, ok(), ok(), ok(), ok(), f32(rows),
                 f32(B + 1), Fake(B + 1, 4, "torch.int32"), B, H, N, N, N, N, d, 0.1, True)
    raises_dtype("seqlens_k", fa.fa_decode_splitkv_varlen, Fake(H * d), Fake(H * 10 * d),
                 Fake(H * 10 * d), Fake(H * d), None, f32(B), B, H, H, 10, d, 2, 0.1)
    # the decode cache and the backward tensors
    raises_dtype("kcache", fa.fa_decode_splitkv_gqa, Fake(H * d), Fake(H * 10 * d, 2, "torch.float16"),
                 Fake(H * 10 * d), Fake(H * d), None, B, H, H, 10, d, 2, 0.1)
    t = lambda: Fake(full)
    raises_dtype("dq", fa.fa_bwd, t(), t(), t(), t(), t(), f32(rows), f32(full), t(), t(),
                 B, H, N, d, 0.1, True)
    raises_dtype("codes", fa.fa_fp8_quantize, t(), f32(d), Fake(full, 2), f32(nsb), B, H, N, d)
    raises_dtype("dout", fa.fa_bwd_varlen, ok(), ok(), ok(), ok(), Fake(full, 2, "torch.float16"),
                 f32(rows), ok(), ok(), ok(), Fake(B + 1, 4, "torch.int32"),
                 Fake(B + 1, 4, "torch.int32"), B, H, N, N, N, N, d, 0.1, True)
