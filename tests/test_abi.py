"""The C-ABI library without a GPU: it loads, exports what include/fa.h
declares, and rejects bad arguments before touching any device."""
import ctypes
import os
import re

import pytest

import exact_attention_116_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x10000          # a 16-byte-aligned fake device address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    return fa.load()


def declared_functions():
    with open(os.path.join(ROOT, "include", "fa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(fa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert fa.fa_status_string(fa.FA_OK) == "FA_OK"
    assert fa.fa_status_string(fa.FA_ERR_WORKSPACE) == "FA_ERR_WORKSPACE"
    assert fa.fa_status_string(99) == "FA_UNKNOWN_STATUS"


def test_params_struct_matches_header():
    # pointer fields, then 2 dtype ints, 4 sizes, float scale, int causal, stream
    assert ctypes.sizeof(fa.fa_fwd_params) == 8 * 8 + 4 * 8 + 8


def _fwd(lib, q=A, k=A, v=A, o=A, lse=A, B=1, H=1, N=16, d=128, scale=0.1, causal=0):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=A + 8), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=-1), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(N=1 << 24), fa.FA_ERR_UNSUPPORTED),      # a 4 GiB head: beyond 32-bit offsets
])
def test_fwd_rejects(lib, kw, status):
    assert _fwd(lib, **kw) == status
    assert fa.fa_last_error() != ""


def test_fwd_ex_rejects(lib):
    assert lib.fa_fwd_ex(None) == fa.FA_ERR_INVALID_ARG
    p = fa.fa_fwd_params(A, A, A, A, A, None, None, None, fa.FA_FP8_E4M3, fa.FA_BF16,
                         1, 1, 64, 128, 0.1, 1, None)
    assert lib.fa_fwd_ex(ctypes.byref(p)) == fa.FA_ERR_INVALID_ARG      # missing scales
    p.q_scale = p.k_scale = p.v_scale = A
    p.d = 64
    assert lib.fa_fwd_ex(ctypes.byref(p)) == fa.FA_ERR_UNSUPPORTED      # fp8 needs d=128
    p.d = 128
    p.out_dtype = fa.FA_FP32
    assert lib.fa_fwd_ex(ctypes.byref(p)) == fa.FA_ERR_UNSUPPORTED      # fp8 writes bf16 only
    p.out_dtype = fa.FA_BF16
    p.k_scale = A + 2
    assert lib.fa_fwd_ex(ctypes.byref(p)) == fa.FA_ERR_INVALID_ARG      # misaligned scales
    p.k_scale = A
    p.in_dtype = fa.FA_BF16
    p.d = 128
    assert lib.fa_fwd_ex(ctypes.byref(p)) == fa.FA_ERR_INVALID_ARG      # scales with bf16
    p.q_scale = p.k_scale = p.v_scale = None
    p.out_dtype = fa.FA_FP8_E4M3
    assert lib.fa_fwd_ex(ctypes.byref(p)) == fa.FA_ERR_INVALID_ARG      # fp8 output
    p.out_dtype = fa.FA_FP32
    p.in_dtype = 7
    assert lib.fa_fwd_ex(ctypes.byref(p)) == fa.FA_ERR_INVALID_ARG
    # 16-bit inputs write o in their own type or in fp32
    p.in_dtype, p.out_dtype = fa.FA_BF16, fa.FA_FP16
    assert lib.fa_fwd_ex(ctypes.byref(p)) == fa.FA_ERR_INVALID_ARG
    p.in_dtype, p.out_dtype = fa.FA_FP16, fa.FA_BF16
    assert lib.fa_fwd_ex(ctypes.byref(p)) == fa.FA_ERR_INVALID_ARG
    p.out_dtype = fa.FA_FP16
    p.d = 96
    assert lib.fa_fwd_ex(ctypes.byref(p)) == fa.FA_ERR_UNSUPPORTED
    p.d = 128
    p.v_scale = A
    assert lib.fa_fwd_ex(ctypes.byref(p)) == fa.FA_ERR_INVALID_ARG      # scales with fp16


def test_workspace_bytes(lib):
    assert fa.fa_decode_workspace_bytes(8, 32, 128, 64) == 8 * 32 * 64 * 129 * 4
    assert fa.fa_decode_workspace_bytes(1, 1, 64, 3) == 1024          # 780 rounded up to 256
    assert fa.fa_decode_workspace_bytes(1, 1, 96, 3) == 0
    assert fa.fa_decode_workspace_bytes(0, 1, 128, 3) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(kc=A + 4), fa.FA_ERR_INVALID_ARG),
    (dict(S=0), fa.FA_ERR_INVALID_ARG),
    (dict(S=17), fa.FA_ERR_INVALID_ARG),     # more splits than keys
    (dict(Lkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=100), fa.FA_ERR_WORKSPACE),
    (dict(Lkv=1 << 24, S=1), fa.FA_ERR_UNSUPPORTED),   # a 4 GiB split
])
def test_decode_ex_rejects(lib, kw, status):
    a = dict(q=A, kc=A, vc=A, o=A, lse=None, B=1, H=2, Lkv=16, d=128, S=4, scale=0.1,
             ws=A, ws_bytes=1 << 20)
    a.update(kw)
    st = lib.fa_decode_splitkv_ex(a["q"], a["kc"], a["vc"], a["o"], a["lse"], a["B"], a["H"],
                                  a["Lkv"], a["d"], a["S"], a["scale"], a["ws"], a["ws_bytes"], None)
    assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=A + 8), fa.FA_ERR_INVALID_ARG),
    (dict(lse=A + 2), fa.FA_ERR_INVALID_ARG),
    (dict(S=0), fa.FA_ERR_INVALID_ARG),
    (dict(S=300, Lkv=200), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    # partials of 8*32*255*129*4 bytes: just past the 32 MiB scratch
    (dict(B=8, H=32, S=255, Lkv=65536), fa.FA_ERR_WORKSPACE),
    (dict(B=1024, H=64, S=1, Lkv=16), fa.FA_ERR_WORKSPACE),
])
def test_decode_noalloc_rejects(lib, kw, status):
    a = dict(q=A, kc=A, vc=A, o=A, lse=None, B=1, H=2, Lkv=16, d=128, S=4, scale=0.1)
    a.update(kw)
    st = lib.fa_decode_splitkv_noalloc(a["q"], a["kc"], a["vc"], a["o"], a["lse"], a["B"], a["H"],
                                       a["Lkv"], a["d"], a["S"], a["scale"], None)
    assert st == status
    assert fa.fa_last_error() != ""


def test_decode_noalloc_limit_matches_header():
    with open(os.path.join(ROOT, "include", "fa.h")) as f:
        m = re.search(r"#define FA_DECODE_SCRATCH_BYTES \((\d+)u << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == fa.FA_DECODE_SCRATCH_BYTES == 32 << 20
    # the largest C4-shaped call that fits: 8 x 32 heads, d = 128, 254 splits
    assert fa.fa_decode_workspace_bytes(8, 32, 128, 254) <= fa.FA_DECODE_SCRATCH_BYTES
    assert fa.fa_decode_workspace_bytes(8, 32, 128, 255) > fa.FA_DECODE_SCRATCH_BYTES


def test_decode_rejects(lib):
    assert lib.fa_decode_splitkv(A, A, A, None, 1, 1, 16, 128, 4) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_decode_splitkv(A, A, A, A, 1, 1, 16, 128, 32) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_decode_splitkv(A, A, A, A, 1, 1, 16, 32, 4) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,status", [
    (dict(Hkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), fa.FA_ERR_INVALID_ARG),      # does not divide Hq = 8
    (dict(Hq=0), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(vc=A + 8), fa.FA_ERR_INVALID_ARG),
    (dict(lse=A + 2), fa.FA_ERR_INVALID_ARG),
    (dict(S=17), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None, ws_bytes=64), fa.FA_ERR_WORKSPACE),
    (dict(ws=A + 4), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=100), fa.FA_ERR_WORKSPACE),
    (dict(Lkv=1 << 24, S=1), fa.FA_ERR_UNSUPPORTED),
])
def test_decode_gqa_rejects(lib, kw, status):
    a = dict(q=A, kc=A, vc=A, o=A, lse=None, B=1, Hq=8, Hkv=2, Lkv=16, d=128, S=4, scale=0.1,
             ws=A, ws_bytes=1 << 20)
    a.update(kw)
    st = lib.fa_decode_splitkv_gqa(a["q"], a["kc"], a["vc"], a["o"], a["lse"], a["B"], a["Hq"],
                                   a["Hkv"], a["Lkv"], a["d"], a["S"], a["scale"], a["ws"],
                                   a["ws_bytes"], None)
    assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=A + 4), fa.FA_ERR_INVALID_ARG),
    (dict(cuq=None), fa.FA_ERR_INVALID_ARG),
    (dict(cuk=A + 2), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(mq=0), fa.FA_ERR_INVALID_ARG),
    (dict(tk=0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(mk=1 << 20, H=32), fa.FA_ERR_UNSUPPORTED),   # 8 GiB of key rows
])
def test_fwd_varlen_rejects(lib, kw, status):
    a = dict(q=A, k=A, v=A, o=A, lse=A, cuq=A, cuk=A, B=2, H=4, mq=64, mk=64, tq=100, tk=100,
             d=128, scale=0.1, causal=1)
    a.update(kw)
    st = lib.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cuq"], a["cuk"], a["B"],
                           a["H"], a["mq"], a["mk"], a["tq"], a["tk"], a["d"], a["scale"],
                           a["causal"], None)
    assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), fa.FA_ERR_INVALID_ARG),
    (dict(codes=A + 8), fa.FA_ERR_INVALID_ARG),
    (dict(scales=None), fa.FA_ERR_INVALID_ARG),
    (dict(signs=A + 1), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
])
def test_fp8_quantize_rejects(lib, kw, status):
    a = dict(x=A, signs=None, codes=A, scales=A, B=1, H=2, N=100, d=128)
    a.update(kw)
    st = lib.fa_fp8_quantize(a["x"], a["signs"], a["codes"], a["scales"], a["B"], a["H"], a["N"],
                             a["d"], None)
    assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(rule=2), fa.FA_ERR_INVALID_ARG),
    (dict(rule=-1), fa.FA_ERR_INVALID_ARG),
    (dict(rule=fa.FA_FP8_SCALE_POW2, x=None), fa.FA_ERR_INVALID_ARG),
    (dict(rule=fa.FA_FP8_SCALE_POW2, d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(rule=fa.FA_FP8_SCALE_AMAX, B=0), fa.FA_ERR_INVALID_ARG),
])
def test_fp8_quantize_ex_rejects(lib, kw, status):
    a = dict(x=A, signs=None, codes=A, scales=A, B=1, H=2, N=100, d=128, rule=0)
    a.update(kw)
    st = lib.fa_fp8_quantize_ex(a["x"], a["signs"], a["codes"], a["scales"], a["B"], a["H"],
                                a["N"], a["d"], a["rule"], None)
    assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(seq=None), fa.FA_ERR_INVALID_ARG),
    (dict(seq=A + 2), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), fa.FA_ERR_INVALID_ARG),
    (dict(S=17), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=A, ws_bytes=64), fa.FA_ERR_WORKSPACE),
])
def test_decode_varlen_rejects(lib, kw, status):
    a = dict(q=A, kc=A, vc=A, o=A, lse=None, seq=A, B=2, Hq=8, Hkv=2, Lkv=16, d=128, S=4,
             scale=0.1, ws=None, ws_bytes=0)
    a.update(kw)
    st = lib.fa_decode_splitkv_varlen(a["q"], a["kc"], a["vc"], a["o"], a["lse"], a["seq"], a["B"],
                                      a["Hq"], a["Hkv"], a["Lkv"], a["d"], a["S"], a["scale"],
                                      a["ws"], a["ws_bytes"], None)
    assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(dq=A + 8), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(N=1 << 24), fa.FA_ERR_UNSUPPORTED),       # a 4 GiB head: beyond 32-bit offsets
    (dict(ws=A, ws_bytes=64), fa.FA_ERR_WORKSPACE),   # smaller than fa_bwd_workspace_bytes
    (dict(ws=None, ws_bytes=64), fa.FA_ERR_WORKSPACE),
    (dict(ws=A + 8, ws_bytes=1 << 20), fa.FA_ERR_WORKSPACE),
    (dict(dtype=fa.FA_FP32), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=fa.FA_FP8_E4M3), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=7), fa.FA_ERR_INVALID_ARG),
])
def test_bwd_rejects(lib, kw, status):
    a = dict(q=A, k=A, v=A, o=A, do=A, lse=A, dq=A, dk=A, dv=A, B=1, H=2, N=100, d=128, scale=0.1,
             causal=1, dtype=fa.FA_BF16, ws=A, ws_bytes=1 << 20)
    a.update(kw)
    args = [a[x] for x in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "B", "H", "N", "d",
                           "scale", "causal")]
    st = lib.fa_bwd_ex(*args, a["dtype"], a["ws"], a["ws_bytes"], None)
    assert st == status
    assert fa.fa_last_error() != ""
    if a["dtype"] == fa.FA_BF16:      # fa_bwd is fa_bwd_ex with FA_BF16
        assert lib.fa_bwd(*args, a["ws"], a["ws_bytes"], None) == status
    assert fa.fa_bwd_workspace_bytes(1, 2, 100) == 2048   # (256 + 200) * 4 rounded up to 256


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(dv=A + 8), fa.FA_ERR_INVALID_ARG),
    (dict(lse=A + 4), fa.FA_ERR_INVALID_ARG),
    (dict(cuq=None), fa.FA_ERR_INVALID_ARG),
    (dict(cuk=A + 2), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(mk=0), fa.FA_ERR_INVALID_ARG),
    (dict(tq=0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(mq=1 << 20, H=32), fa.FA_ERR_UNSUPPORTED),   # 8 GiB of query rows
    (dict(ws=A, ws_bytes=64), fa.FA_ERR_WORKSPACE),     # smaller than fa_bwd_workspace_bytes(1, H, tq)
    (dict(ws=None, ws_bytes=64), fa.FA_ERR_WORKSPACE),
    (dict(ws=A + 8, ws_bytes=1 << 20), fa.FA_ERR_WORKSPACE),
])
def test_bwd_varlen_rejects(lib, kw, status):
    a = dict(q=A, k=A, v=A, o=A, do=A, lse=A, dq=A, dk=A, dv=A, cuq=A, cuk=A, B=2, H=4, mq=64,
             mk=80, tq=100, tk=150, d=128, scale=0.1, causal=1, ws=A, ws_bytes=1 << 20)
    a.update(kw)
    st = lib.fa_bwd_varlen(*[a[x] for x in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "cuq",
                                            "cuk", "B", "H", "mq", "mk", "tq", "tk", "d", "scale",
                                            "causal", "ws", "ws_bytes")], None)
    assert st == status
    assert fa.fa_last_error() != ""
    # D takes H * total_q fp32 values: the dense workspace of one batch of total_q rows
    assert fa.fa_bwd_workspace_bytes(1, 4, 100) == 3584   # (448 + 400) * 4 rounded up to 256
    # two fp32 row arrays, the second 256-byte aligned after the first
    for B, H, N in ((1, 1, 1), (2, 3, 65), (4, 16, 8192), (1, 32, 14072)):
        rows = B * H * N
        nb = fa.fa_bwd_workspace_bytes(B, H, N)
        assert nb % 256 == 0 and nb >= (-(-rows // 64) * 64 + rows) * 4


def test_binding_rejects_host_and_strided_tensors():
    import torch
    x = torch.zeros(1, 1, 16, 128, dtype=torch.bfloat16)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd(x, x, x, x, x, 1, 1, 16, 128, 0.1, False)
    assert e.value.status == fa.FA_ERR_INVALID_ARG and "GPU" in str(e.value)

    class FakeDevice:   # a GPU tensor stand-in that is not contiguous
        is_cuda = True

        def is_contiguous(self):
            return False

        def data_ptr(self):
            return A
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd(FakeDevice(), A, A, A, A, 1, 1, 16, 128, 0.1, False)
    assert "contiguous" in str(e.value)


def test_binding_raises_with_status():
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd(A, A, A, A, None, 1, 1, 16, 128, 0.1, False)
    assert e.value.status == fa.FA_ERR_INVALID_ARG and "lse" in str(e.value)
