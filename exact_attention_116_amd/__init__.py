"""Exact attention on AMD Instinct MI355X: Python binding of ``libfa.so``.

The functions below have the names and arguments of the C entry points in
``include/fa.h`` and only marshal arguments (device pointers from tensors or
integers, sizes, the stream handle).  Every step of the computation runs in
the library's HIP kernels; when the library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)
FA_BF16, FA_FP32, FA_FP8_E4M3, FA_FP16 = range(4)
FA_FP8_SCALE_AMAX, FA_FP8_SCALE_POW2 = range(2)
FA_DECODE_SCRATCH_BYTES = 32 << 20   # the fixed scratch of fa_decode_splitkv_noalloc

EXPORTS = ("fa_fwd", "fa_fwd_ex", "fa_decode_splitkv", "fa_decode_workspace_bytes",
           "fa_decode_splitkv_ex", "fa_decode_splitkv_noalloc", "fa_decode_splitkv_gqa",
           "fa_decode_splitkv_varlen",
           "fa_fwd_varlen", "fa_fp8_quantize", "fa_fp8_quantize_ex",
           "fa_bwd_workspace_bytes", "fa_bwd", "fa_bwd_ex", "fa_bwd_varlen",
           "fa_status_string", "fa_last_error")


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class fa_fwd_params(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("q_scale", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p),
                ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("B", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int), ("d", ctypes.c_int),
                ("scale", ctypes.c_float), ("causal", ctypes.c_int), ("stream", ctypes.c_void_p)]


_lib = None


def load(path: str | None = None):
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise FaError(-1, f"{path} is missing: build it with `python -m exact_attention_116_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, F, I]
    lib.fa_fwd.restype = I
    lib.fa_fwd_ex.argtypes = [ctypes.POINTER(fa_fwd_params)]
    lib.fa_fwd_ex.restype = I
    lib.fa_decode_splitkv.argtypes = [P, P, P, P, I, I, I, I, I]
    lib.fa_decode_splitkv.restype = I
    lib.fa_decode_workspace_bytes.argtypes = [I, I, I, I]
    lib.fa_decode_workspace_bytes.restype = Z
    lib.fa_decode_splitkv_ex.argtypes = [P, P, P, P, P, I, I, I, I, I, F, P, Z, P]
    lib.fa_decode_splitkv_ex.restype = I
    lib.fa_decode_splitkv_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, F, P]
    lib.fa_decode_splitkv_noalloc.restype = I
    lib.fa_decode_splitkv_gqa.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, P, Z, P]
    lib.fa_decode_splitkv_gqa.restype = I
    lib.fa_decode_splitkv_varlen.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, P, Z, P]
    lib.fa_decode_splitkv_varlen.restype = I
    lib.fa_fwd_varlen.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P]
    lib.fa_fwd_varlen.restype = I
    lib.fa_fp8_quantize.argtypes = [P, P, P, P, I, I, I, I, P]
    lib.fa_fp8_quantize.restype = I
    lib.fa_fp8_quantize_ex.argtypes = [P, P, P, P, I, I, I, I, I, P]
    lib.fa_fp8_quantize_ex.restype = I
    lib.fa_bwd_workspace_bytes.argtypes = [I, I, I]
    lib.fa_bwd_workspace_bytes.restype = Z
    lib.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, P, Z, P]
    lib.fa_bwd.restype = I
    lib.fa_bwd_ex.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, I, P, Z, P]
    lib.fa_bwd_ex.restype = I
    lib.fa_bwd_varlen.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P, Z, P]
    lib.fa_bwd_varlen.restype = I
    lib.fa_status_string.argtypes = [I]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


# torch dtype names accepted for each kind of tensor argument
BF16, F16, F32, I32 = ("torch.bfloat16",), ("torch.float16",), ("torch.float32",), ("torch.int32",)
U8 = ("torch.uint8", "torch.int8", "torch.float8_e4m3fn")   # E4M3FN codes as bytes
_IN_DT = {0: BF16, 3: F16, 2: U8}          # FA_BF16, FA_FP16, FA_FP8_E4M3
_OUT_DT = {0: BF16, 3: F16, 1: F32}        # FA_BF16, FA_FP16, FA_FP32


def _ptr(x, nbytes: int = 0, name: str = "tensor", dtypes=None):
    """Device address of a tensor (``data_ptr()``), an int (taken as a device
    address as is), or None.  A tensor must live on a GPU, be contiguous,
    hold at least ``nbytes`` bytes and, when ``dtypes`` is given, have one of
    those dtypes: the kernels read and write the dense layouts and element
    types ``include/fa.h`` states, and a host address, a short buffer or
    another element type handed to a kernel would fault the device or be
    read as the wrong numbers.  The C entry points see plain pointers and
    cannot check any of this; this is where it is checked."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise FaError(FA_ERR_INVALID_ARG, "tensor arguments must be GPU tensors")
    if not x.is_contiguous():
        raise FaError(FA_ERR_INVALID_ARG, "tensor arguments must be contiguous")
    have = x.numel() * x.element_size()
    if nbytes > 0 and have < nbytes:
        raise FaError(FA_ERR_INVALID_ARG, f"{name} holds {have} bytes; the call needs {nbytes}")
    if dtypes is not None and str(x.dtype) not in dtypes:
        raise FaError(FA_ERR_INVALID_ARG, f"{name} has dtype {x.dtype}; the call needs "
                                          f"{' or '.join(dtypes)}")
    return x.data_ptr()


def _n(*dims) -> int:
    """Product of the dimensions (0 if any is negative: the library rejects those)."""
    r = 1
    for v in dims:
        v = int(v)
        if v < 0:
            return 0
        r *= v
    return r


_IN_BYTES = {FA_BF16: 2, FA_FP16: 2, FA_FP8_E4M3: 1}
_OUT_BYTES = {FA_BF16: 2, FA_FP16: 2, FA_FP32: 4}


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int, what: str):
    if status != FA_OK:
        lib = load()
        raise FaError(status, f"{what}: {lib.fa_status_string(status).decode()}: "
                              f"{lib.fa_last_error().decode()}")


def fa_status_string(status: int) -> str:
    return load().fa_status_string(status).decode()


def fa_last_error() -> str:
    return load().fa_last_error().decode()


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal):
    """bf16 [B,H,N,d] q, k, v -> bf16 o, fp32 lse [B,H,N]; default stream."""
    t, r = 2 * _n(B, H, N, d), 4 * _n(B, H, N)
    _check(load().fa_fwd(_ptr(q, t, "q", BF16), _ptr(k, t, "k", BF16), _ptr(v, t, "v", BF16),
                         _ptr(o, t, "o", BF16), _ptr(lse, r, "lse", F32), B, H, N, d, float(scale),
                         int(bool(causal))), "fa_fwd")


def fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, in_dtype=FA_BF16, out_dtype=FA_BF16,
              q_scale=None, k_scale=None, v_scale=None, stream=None):
    t = _IN_BYTES.get(in_dtype, 0) * _n(B, H, N, d)
    to = _OUT_BYTES.get(out_dtype, 0) * _n(B, H, N, d)
    sc = 4 * _n(B, H, (int(N) + 63) // 64)
    di, do_ = _IN_DT.get(in_dtype), _OUT_DT.get(out_dtype)
    p = fa_fwd_params(_ptr(q, t, "q", di), _ptr(k, t, "k", di), _ptr(v, t, "v", di),
                      _ptr(o, to, "o", do_), _ptr(lse, 4 * _n(B, H, N), "lse", F32),
                      _ptr(q_scale, sc, "q_scale", F32), _ptr(k_scale, sc, "k_scale", F32),
                      _ptr(v_scale, sc, "v_scale", F32), in_dtype, out_dtype, B, H, N, d,
                      float(scale), int(bool(causal)), _stream(stream))
    _check(load().fa_fwd_ex(ctypes.byref(p)), "fa_fwd_ex")


def fa_decode_splitkv(q, kcache, vcache, o, B, H, Lkv, d, num_splits):
    t, c = 2 * _n(B, H, d), 2 * _n(B, H, Lkv, d)
    _check(load().fa_decode_splitkv(_ptr(q, t, "q", BF16), _ptr(kcache, c, "kcache", BF16),
                                    _ptr(vcache, c, "vcache", BF16), _ptr(o, t, "o", BF16), B, H,
                                    Lkv, d, num_splits), "fa_decode_splitkv")


def fa_decode_workspace_bytes(B, H, d, num_splits) -> int:
    return int(load().fa_decode_workspace_bytes(B, H, d, num_splits))


def fa_decode_splitkv_ex(q, kcache, vcache, o, lse, B, H, Lkv, d, num_splits, scale, workspace,
                         workspace_bytes, stream=None):
    t, c = 2 * _n(B, H, d), 2 * _n(B, H, Lkv, d)
    _check(load().fa_decode_splitkv_ex(_ptr(q, t, "q", BF16), _ptr(kcache, c, "kcache", BF16),
                                       _ptr(vcache, c, "vcache", BF16), _ptr(o, t, "o", BF16),
                                       _ptr(lse, 4 * _n(B, H), "lse", F32), B, H, Lkv, d, num_splits,
                                       float(scale), _ptr(workspace, int(workspace_bytes), "workspace"),
                                       int(workspace_bytes), _stream(stream)),
           "fa_decode_splitkv_ex")


def fa_decode_splitkv_noalloc(q, kcache, vcache, o, lse, B, H, Lkv, d, num_splits, scale,
                              stream=None):
    """fa_decode_splitkv_ex without a workspace: the partials go to the
    library's fixed scratch (at most FA_DECODE_SCRATCH_BYTES), so the call
    allocates nothing.  Calls that overlap on one GPU share that scratch."""
    t, c = 2 * _n(B, H, d), 2 * _n(B, H, Lkv, d)
    _check(load().fa_decode_splitkv_noalloc(_ptr(q, t, "q", BF16), _ptr(kcache, c, "kcache", BF16),
                                            _ptr(vcache, c, "vcache", BF16), _ptr(o, t, "o", BF16),
                                            _ptr(lse, 4 * _n(B, H), "lse", F32), B, H, Lkv, d,
                                            num_splits, float(scale), _stream(stream)),
           "fa_decode_splitkv_noalloc")


def fa_decode_splitkv_gqa(q, kcache, vcache, o, lse, B, Hq, Hkv, Lkv, d, num_splits, scale,
                          workspace=None, workspace_bytes=0, stream=None):
    """Grouped K/V heads: q, o bf16 [B,Hq,1,d]; caches bf16 [B,Hkv,Lkv,d]."""
    t, c = 2 * _n(B, Hq, d), 2 * _n(B, Hkv, Lkv, d)
    _check(load().fa_decode_splitkv_gqa(_ptr(q, t, "q", BF16), _ptr(kcache, c, "kcache", BF16),
                                        _ptr(vcache, c, "vcache", BF16), _ptr(o, t, "o", BF16),
                                        _ptr(lse, 4 * _n(B, Hq), "lse", F32), B, Hq, Hkv, Lkv, d,
                                        num_splits, float(scale),
                                        _ptr(workspace, int(workspace_bytes), "workspace"),
                                        int(workspace_bytes), _stream(stream)),
           "fa_decode_splitkv_gqa")


def fa_bwd_workspace_bytes(B, H, N) -> int:
    return int(load().fa_bwd_workspace_bytes(B, H, N))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, workspace=None,
           workspace_bytes=0, stream=None):
    """bf16 [B,H,N,d] q, k, v, o, dout and fp32 lse [B,H,N] -> bf16 dq, dk, dv."""
    t, r = 2 * _n(B, H, N, d), 4 * _n(B, H, N)
    _check(load().fa_bwd(_ptr(q, t, "q", BF16), _ptr(k, t, "k", BF16), _ptr(v, t, "v", BF16),
                         _ptr(o, t, "o", BF16), _ptr(dout, t, "dout", BF16), _ptr(lse, r, "lse", F32),
                         _ptr(dq, t, "dq", BF16), _ptr(dk, t, "dk", BF16), _ptr(dv, t, "dv", BF16),
                         B, H, N, d, float(scale),
                         int(bool(causal)), _ptr(workspace, int(workspace_bytes), "workspace"),
                         int(workspace_bytes), _stream(stream)), "fa_bwd")


def fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype=FA_BF16,
              workspace=None, workspace_bytes=0, stream=None):
    """fa_bwd with the tensor type as an argument: FA_BF16 or FA_FP16."""
    t, r = 2 * _n(B, H, N, d), 4 * _n(B, H, N)
    dt = {FA_BF16: BF16, FA_FP16: F16}.get(int(dtype))
    _check(load().fa_bwd_ex(_ptr(q, t, "q", dt), _ptr(k, t, "k", dt), _ptr(v, t, "v", dt),
                            _ptr(o, t, "o", dt), _ptr(dout, t, "dout", dt), _ptr(lse, r, "lse", F32),
                            _ptr(dq, t, "dq", dt), _ptr(dk, t, "dk", dt), _ptr(dv, t, "dv", dt),
                            B, H, N, d, float(scale),
                            int(bool(causal)), int(dtype),
                            _ptr(workspace, int(workspace_bytes), "workspace"),
                            int(workspace_bytes), _stream(stream)),
           "fa_bwd_ex")


def fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, B, H,
                  max_seqlen_q, max_seqlen_k, total_q, total_k, d, scale, causal, workspace=None,
                  workspace_bytes=0, stream=None):
    """Packed bf16 q, o, dout, dq [total_q,H,d], k, v, dk, dv [total_k,H,d] and fp32
    lse [H,total_q] (fa_fwd_varlen's outputs) -> bf16 dq, dk, dv."""
    tq, tk, cu = 2 * _n(total_q, H, d), 2 * _n(total_k, H, d), 4 * _n(int(B) + 1)
    _check(load().fa_bwd_varlen(_ptr(q, tq, "q", BF16), _ptr(k, tk, "k", BF16),
                                _ptr(v, tk, "v", BF16), _ptr(o, tq, "o", BF16),
                                _ptr(dout, tq, "dout", BF16), _ptr(lse, 4 * _n(H, total_q), "lse", F32),
                                _ptr(dq, tq, "dq", BF16), _ptr(dk, tk, "dk", BF16),
                                _ptr(dv, tk, "dv", BF16),
                                _ptr(cu_seqlens_q, cu, "cu_seqlens_q", I32),
                                _ptr(cu_seqlens_k, cu, "cu_seqlens_k", I32), B, H, max_seqlen_q,
                                max_seqlen_k, total_q, total_k, d, float(scale), int(bool(causal)),
                                _ptr(workspace, int(workspace_bytes), "workspace"),
                                int(workspace_bytes), _stream(stream)), "fa_bwd_varlen")


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, max_seqlen_q, max_seqlen_k,
                  total_q, total_k, d, scale, causal, stream=None):
    """Packed bf16 q [total_q,H,d], k, v [total_k,H,d] -> o, fp32 lse [H,total_q]."""
    tq, tk, cu = 2 * _n(total_q, H, d), 2 * _n(total_k, H, d), 4 * _n(int(B) + 1)
    _check(load().fa_fwd_varlen(_ptr(q, tq, "q", BF16), _ptr(k, tk, "k", BF16),
                                _ptr(v, tk, "v", BF16), _ptr(o, tq, "o", BF16),
                                _ptr(lse, 4 * _n(H, total_q), "lse", F32),
                                _ptr(cu_seqlens_q, cu, "cu_seqlens_q", I32),
                                _ptr(cu_seqlens_k, cu, "cu_seqlens_k", I32), B, H, max_seqlen_q,
                                max_seqlen_k, total_q, total_k, d, float(scale),
                                int(bool(causal)), _stream(stream)), "fa_fwd_varlen")


def fa_fp8_quantize(x, signs, codes, scales, B, H, N, d, stream=None, scale_rule=None):
    """bf16 [B,H,N,d] -> E4M3FN codes + fp32 [B,H,ceil(N/64)] scales; signs [d] rotates.
    ``scale_rule`` FA_FP8_SCALE_AMAX (max|x| / 448, the default) or
    FA_FP8_SCALE_POW2 (the smallest power of two with max|x| / scale <= 448)."""
    args = (_ptr(x, 2 * _n(B, H, N, d), "x", BF16), _ptr(signs, 4 * _n(d), "signs", F32),
            _ptr(codes, _n(B, H, N, d), "codes", U8),
            _ptr(scales, 4 * _n(B, H, (int(N) + 63) // 64), "scales", F32), B, H, N, d)
    if scale_rule is None:
        _check(load().fa_fp8_quantize(*args, _stream(stream)), "fa_fp8_quantize")
    else:
        _check(load().fa_fp8_quantize_ex(*args, int(scale_rule), _stream(stream)),
               "fa_fp8_quantize_ex")


def fa_decode_splitkv_varlen(q, kcache, vcache, o, lse, seqlens_k, B, Hq, Hkv, Lkv, d, num_splits,
                             scale, workspace=None, workspace_bytes=0, stream=None):
    """Grouped decode over padded caches [B,Hkv,Lkv,d] with int32 seqlens_k [B] (device)."""
    t, c = 2 * _n(B, Hq, d), 2 * _n(B, Hkv, Lkv, d)
    _check(load().fa_decode_splitkv_varlen(_ptr(q, t, "q", BF16), _ptr(kcache, c, "kcache", BF16),
                                           _ptr(vcache, c, "vcache", BF16), _ptr(o, t, "o", BF16),
                                           _ptr(lse, 4 * _n(B, Hq), "lse", F32),
                                           _ptr(seqlens_k, 4 * _n(B), "seqlens_k", I32), B, Hq, Hkv,
                                           Lkv, d, num_splits, float(scale),
                                           _ptr(workspace, int(workspace_bytes), "workspace"),
                                           int(workspace_bytes), _stream(stream)),
           "fa_decode_splitkv_varlen")
