// C-ABI host layer of the attention library: argument validation, the
// library-owned workspace (decode partials, backward row sums; released when
// the library is unloaded) and dispatch to the HIP launchers.
// Every check runs before any HIP call, so a rejected call touches no device.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/fa.h"
#include "fa_internal.h"

static_assert(fa::kDecodeScratchBytes == (size_t)FA_DECODE_SCRATCH_BYTES,
              "the fixed decode scratch has the size fa.h states");

namespace {

thread_local std::string g_last_error;

fa_status fail(fa_status s, const char* what) {
  g_last_error = what;
  return s;
}

fa_status hip_fail(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return FA_ERR_HIP;
}

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool good_scale(float s) { return std::isfinite(s) && s > 0.f; }

constexpr double kLog2e = 1.4426950408889634074;

fa_status check_fwd(const fa_fwd_params* p) {
  if (!p) return fail(FA_ERR_INVALID_ARG, "params is NULL");
  if (!aligned16(p->q) || !aligned16(p->k) || !aligned16(p->v) || !aligned16(p->o) ||
      !aligned16(p->lse))
    return fail(FA_ERR_INVALID_ARG, "q, k, v, o and lse must be non-NULL and 16-byte aligned");
  if (p->B < 1 || p->H < 1 || p->N < 1)
    return fail(FA_ERR_INVALID_ARG, "B, H and N must be >= 1");
  if (p->d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1");
  if (!good_scale(p->scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (p->out_dtype != FA_BF16 && p->out_dtype != FA_FP32 && p->out_dtype != FA_FP16)
    return fail(FA_ERR_INVALID_ARG, "out_dtype must be FA_BF16, FA_FP16 or FA_FP32");
  const long long elems = (long long)p->B * p->H * p->N * p->d;
  if ((long long)p->B * p->H * ((p->N + 31) / 32) > 0x7FFFFFFFLL || elems <= 0)
    return fail(FA_ERR_INVALID_ARG, "problem too large for one launch");
  // the kernels address one head with 32-bit byte offsets
  const long long elem_bytes = p->in_dtype == FA_FP8_E4M3 ? 1 : 2;
  if ((long long)p->N * p->d * elem_bytes >= (1LL << 32))
    return fail(FA_ERR_UNSUPPORTED, "one (batch, head) slice must be smaller than 4 GiB");
  if (p->in_dtype == FA_BF16 || p->in_dtype == FA_FP16) {
    if (p->q_scale || p->k_scale || p->v_scale)
      return fail(FA_ERR_INVALID_ARG, "block scales are only accepted with FA_FP8_E4M3 inputs");
    if (p->out_dtype != FA_FP32 && p->out_dtype != p->in_dtype)
      return fail(FA_ERR_INVALID_ARG, "16-bit inputs write o in their own type or in fp32");
    if (p->d != 64 && p->d != 128) return fail(FA_ERR_UNSUPPORTED, "16-bit path supports d = 64 or 128");
    return FA_OK;
  }
  if (p->in_dtype == FA_FP8_E4M3) {
    if (!p->q_scale || !p->k_scale || !p->v_scale)
      return fail(FA_ERR_INVALID_ARG, "fp8 inputs need q_scale, k_scale and v_scale");
    if ((reinterpret_cast<uintptr_t>(p->q_scale) | reinterpret_cast<uintptr_t>(p->k_scale) |
         reinterpret_cast<uintptr_t>(p->v_scale)) & 3u)
      return fail(FA_ERR_INVALID_ARG, "block scales must be 4-byte aligned");
    if (p->d != 128) return fail(FA_ERR_UNSUPPORTED, "fp8 path supports d = 128");
    if (p->out_dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "fp8 path writes bf16 output");
    return FA_OK;
  }
  return fail(FA_ERR_INVALID_ARG, "in_dtype must be FA_BF16, FA_FP16 or FA_FP8_E4M3");
}

fa_status run_fwd(const fa_fwd_params* p) {
  fa_status st = check_fwd(p);
  if (st != FA_OK) return st;
  fa::FwdArgs a{};
  a.q = p->q; a.k = p->k; a.v = p->v; a.o = p->o; a.lse = p->lse;
  a.q_scale = p->q_scale; a.k_scale = p->k_scale; a.v_scale = p->v_scale;
  a.B = p->B; a.H = p->H; a.N = p->N; a.d = p->d;
  a.scale = p->scale;
  a.scale_log2 = (float)((double)p->scale * kLog2e);
  a.causal = p->causal != 0;
  a.out_f32 = p->out_dtype == FA_FP32;
  a.in_f16 = p->in_dtype == FA_FP16;
  a.stream = p->stream;
  a.cu_q = nullptr;
  a.cu_k = nullptr;
  a.Nk = p->N;
  hipError_t e = (p->in_dtype == FA_FP8_E4M3) ? fa::launch_fwd_fp8(a) : fa::launch_fwd_bf16(a);
  if (e == hipErrorNotSupported) return fail(FA_ERR_UNSUPPORTED, "no kernel for this request");
  if (e != hipSuccess) return hip_fail(e, "fa_fwd launch");
  g_last_error.clear();
  return FA_OK;
}

size_t decode_ws_bytes(int B, int H, int d, int S) {
  const size_t n = (size_t)B * H * S * (size_t)(d + 1) * 4u;
  return (n + 255u) & ~(size_t)255u;
}

fa_status check_decode(const void* q, const void* kc, const void* vc, const void* o, int B, int H,
                       int Lkv, int d, int S, float scale) {
  if (!aligned16(q) || !aligned16(kc) || !aligned16(vc) || !aligned16(o))
    return fail(FA_ERR_INVALID_ARG, "q, kcache, vcache and o must be non-NULL and 16-byte aligned");
  if (B < 1 || H < 1 || Lkv < 1) return fail(FA_ERR_INVALID_ARG, "B, H and Lkv must be >= 1");
  if (S < 1 || S > Lkv) return fail(FA_ERR_INVALID_ARG, "num_splits must be in [1, Lkv]");
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1");
  if (!good_scale(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "decode supports d = 64 or 128");
  if ((long long)B * H * S > 0x7FFFFFFFLL) return fail(FA_ERR_INVALID_ARG, "B*H*num_splits too large");
  // a split is addressed with 32-bit byte offsets
  const long long chunk = ((long long)Lkv + S - 1) / S;
  if (chunk * d * 2 >= (1LL << 32))
    return fail(FA_ERR_UNSUPPORTED, "one split of the KV cache must be smaller than 4 GiB");
  return FA_OK;
}

// Hkv = 0: plain multi-head decode (one K/V head per query head);
// Hkv > 0: grouped heads, query head h reads K/V head h / (H / Hkv), and an
// optional length per sequence (seqlens, device, or null).
fa_status run_decode(const void* q, const void* kc, const void* vc, void* o, float* lse, int B,
                     int H, int Hkv, int Lkv, int d, int S, float scale, void* ws, void* stream,
                     const int* seqlens = nullptr) {
  fa::DecodeArgs a{};
  a.q = q; a.k = kc; a.v = vc; a.o = o; a.lse = lse;
  a.part_o = static_cast<float*>(ws);
  a.part_lse = static_cast<float*>(ws) + (size_t)B * H * S * d;
  a.B = B; a.H = H; a.Lkv = Lkv; a.d = d; a.num_splits = S;
  a.Hkv = Hkv > 0 ? Hkv : H;
  a.seqlens_k = seqlens;
  a.scale_log2 = (float)((double)scale * kLog2e);
  a.stream = stream;
  hipError_t e = Hkv > 0 ? fa::launch_decode_gqa(a) : fa::launch_decode(a);
  if (e != hipSuccess) return hip_fail(e, Hkv > 0 ? "fa_decode_splitkv_gqa launch" : "fa_decode_splitkv launch");
  g_last_error.clear();
  return FA_OK;
}

// Library-owned decode workspace: one buffer per device, grown on demand and
// released when the library is unloaded (dlclose, or the end of the process).
struct OwnedWorkspace {
  std::mutex mu;
  std::vector<void*> ptr;
  std::vector<size_t> bytes;
  ~OwnedWorkspace() {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) cur = -1;
    for (size_t d = 0; d < ptr.size(); ++d) {
      if (!ptr[d]) continue;
      (void)hipSetDevice((int)d);   // free each buffer with its own device current
      (void)hipFree(ptr[d]);
      ptr[d] = nullptr;
    }
    if (cur >= 0) (void)hipSetDevice(cur);
  }
};
OwnedWorkspace g_ws;

// The current device's library-owned workspace, at least `need` bytes.  On
// success `lock` holds the workspace mutex; the caller keeps it until the
// launch that uses the buffer is queued, so that no other thread can grow
// (free and reallocate) the buffer in between.
fa_status owned_workspace(size_t need, void** out, std::unique_lock<std::mutex>& lock) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  lock = std::unique_lock<std::mutex>(g_ws.mu);
  if ((int)g_ws.ptr.size() <= dev) {
    g_ws.ptr.resize(dev + 1, nullptr);
    g_ws.bytes.resize(dev + 1, 0);
  }
  if (g_ws.bytes[dev] < need) {
    if (g_ws.ptr[dev]) {
      // the old buffer may still be read by queued work of an earlier call
      e = hipDeviceSynchronize();
      if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
      (void)hipFree(g_ws.ptr[dev]);  // the buffer is dropped either way
      g_ws.ptr[dev] = nullptr;
      g_ws.bytes[dev] = 0;
    }
    e = hipMalloc(&g_ws.ptr[dev], need);
    if (e != hipSuccess) {
      g_ws.ptr[dev] = nullptr;
      return fail(FA_ERR_WORKSPACE, "could not allocate the library-owned workspace");
    }
    g_ws.bytes[dev] = need;
  }
  *out = g_ws.ptr[dev];
  return FA_OK;
}

// The grouped-head decode behind fa_decode_splitkv_gqa and
// fa_decode_splitkv_varlen (seqlens may be null).
fa_status decode_grouped(const void* q, const void* kcache, const void* vcache, void* o,
                         float* lse, const int* seqlens, int B, int Hq, int Hkv, int Lkv, int d,
                         int num_splits, float scale, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (Hkv < 1 || Hq < 1 || Hq % Hkv != 0)
    return fail(FA_ERR_INVALID_ARG, "Hkv must be >= 1 and divide Hq");
  fa_status st = check_decode(q, kcache, vcache, o, B, Hq, Lkv, d, num_splits, scale);
  if (st != FA_OK) return st;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const size_t need = decode_ws_bytes(B, Hq, d, num_splits);
  void* ws = workspace;
  std::unique_lock<std::mutex> ws_lock;   // held through the launch when ws is library-owned
  if (!workspace) {
    if (workspace_bytes != 0) return fail(FA_ERR_WORKSPACE, "workspace is NULL but workspace_bytes is not 0");
    st = owned_workspace(need, &ws, ws_lock);
    if (st != FA_OK) return st;
  } else {
    if (!aligned16(workspace)) return fail(FA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE, "workspace smaller than fa_decode_workspace_bytes()");
  }
  return run_decode(q, kcache, vcache, o, lse, B, Hq, Hkv, Lkv, d, num_splits, scale, ws, stream,
                    seqlens);
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal) {
  fa_fwd_params p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.in_dtype = FA_BF16;
  p.out_dtype = FA_BF16;
  p.B = B; p.H = H; p.N = N; p.d = d;
  p.scale = scale;
  p.causal = causal;
  p.stream = nullptr;
  return run_fwd(&p);
}

fa_status fa_fwd_ex(const fa_fwd_params* p) { return run_fwd(p); }

size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits) {
  if (B < 1 || H < 1 || num_splits < 1 || (d != 64 && d != 128)) return 0;
  return decode_ws_bytes(B, H, d, num_splits);
}

fa_status fa_decode_splitkv_ex(const void* q, const void* kcache, const void* vcache, void* o,
                               float* lse, int B, int H, int Lkv, int d, int num_splits,
                               float scale, void* workspace, size_t workspace_bytes,
                               void* stream) {
  fa_status st = check_decode(q, kcache, vcache, o, B, H, Lkv, d, num_splits, scale);
  if (st != FA_OK) return st;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (!aligned16(workspace)) return fail(FA_ERR_WORKSPACE, "workspace must be non-NULL and 16-byte aligned");
  if (workspace_bytes < decode_ws_bytes(B, H, d, num_splits))
    return fail(FA_ERR_WORKSPACE, "workspace smaller than fa_decode_workspace_bytes()");
  return run_decode(q, kcache, vcache, o, lse, B, H, 0, Lkv, d, num_splits, scale, workspace, stream);
}

fa_status fa_decode_splitkv(const void* q, const void* kcache, const void* vcache, void* o, int B,
                            int H, int Lkv, int d, int num_splits) {
  const float scale = d > 0 ? (float)(1.0 / std::sqrt((double)d)) : 0.f;
  fa_status st = check_decode(q, kcache, vcache, o, B, H, Lkv, d, num_splits, scale);
  if (st != FA_OK) return st;
  void* ws = nullptr;
  std::unique_lock<std::mutex> ws_lock;   // held through the launch
  st = owned_workspace(decode_ws_bytes(B, H, d, num_splits), &ws, ws_lock);
  if (st != FA_OK) return st;
  return run_decode(q, kcache, vcache, o, nullptr, B, H, 0, Lkv, d, num_splits, scale, ws, nullptr);
}

fa_status fa_decode_splitkv_noalloc(const void* q, const void* kcache, const void* vcache, void* o,
                                    float* lse, int B, int H, int Lkv, int d, int num_splits,
                                    float scale, void* stream) {
  fa_status st = check_decode(q, kcache, vcache, o, B, H, Lkv, d, num_splits, scale);
  if (st != FA_OK) return st;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (decode_ws_bytes(B, H, d, num_splits) > (size_t)FA_DECODE_SCRATCH_BYTES)
    return fail(FA_ERR_WORKSPACE,
                "B*H*num_splits*(d+1)*4 bytes of partials exceed FA_DECODE_SCRATCH_BYTES (32 MiB)");
  void* ws = nullptr;
  hipError_t e = fa::decode_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "fa_decode_splitkv_noalloc scratch lookup");
  return run_decode(q, kcache, vcache, o, lse, B, H, 0, Lkv, d, num_splits, scale, ws, stream);
}

fa_status fa_decode_splitkv_gqa(const void* q, const void* kcache, const void* vcache, void* o,
                                float* lse, int B, int Hq, int Hkv, int Lkv, int d, int num_splits,
                                float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_grouped(q, kcache, vcache, o, lse, nullptr, B, Hq, Hkv, Lkv, d, num_splits, scale,
                        workspace, workspace_bytes, stream);
}

fa_status fa_decode_splitkv_varlen(const void* q, const void* kcache, const void* vcache, void* o,
                                   float* lse, const int* seqlens_k, int B, int Hq, int Hkv,
                                   int Lkv, int d, int num_splits, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!seqlens_k || (reinterpret_cast<uintptr_t>(seqlens_k) & 3u))
    return fail(FA_ERR_INVALID_ARG, "seqlens_k must be non-NULL and 4-byte aligned");
  return decode_grouped(q, kcache, vcache, o, lse, seqlens_k, B, Hq, Hkv, Lkv, d, num_splits,
                        scale, workspace, workspace_bytes, stream);
}



fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                        int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int d,
                        float scale, int causal, void* stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return fail(FA_ERR_INVALID_ARG, "q, k, v, o and lse must be non-NULL and 16-byte aligned");
  if (!cu_seqlens_q || !cu_seqlens_k ||
      ((reinterpret_cast<uintptr_t>(cu_seqlens_q) | reinterpret_cast<uintptr_t>(cu_seqlens_k)) & 3u))
    return fail(FA_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must be non-NULL and 4-byte aligned");
  if (B < 1 || H < 1) return fail(FA_ERR_INVALID_ARG, "B and H must be >= 1");
  if (max_seqlen_q < 1 || max_seqlen_k < 1 || total_q < 1 || total_k < 1)
    return fail(FA_ERR_INVALID_ARG, "max_seqlen_q, max_seqlen_k, total_q and total_k must be >= 1");
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1");
  if (!good_scale(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "varlen path supports d = 64 or 128");
  if ((long long)B * H * ((max_seqlen_q + 255) / 256) > 0x7FFFFFFFLL)
    return fail(FA_ERR_INVALID_ARG, "problem too large for one launch");
  // one sequence of one head is addressed with 32-bit byte offsets over its rows
  const long long row_bytes = (long long)H * d * 2;
  if ((long long)max_seqlen_q * row_bytes >= (1LL << 32) || (long long)max_seqlen_k * row_bytes >= (1LL << 32))
    return fail(FA_ERR_UNSUPPORTED, "one sequence must span under 4 GiB of rows");
  fa::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.N = max_seqlen_q; a.d = d;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * kLog2e);
  a.causal = causal ? 1 : 0;
  a.out_f32 = 0;
  a.stream = stream;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.Nk = max_seqlen_k;
  a.total_q = total_q;
  a.total_k = total_k;
  hipError_t e = fa::launch_fwd_bf16(a);
  if (e != hipSuccess) return hip_fail(e, "fa_fwd_varlen launch");
  g_last_error.clear();
  return FA_OK;
}

fa_status fa_fp8_quantize(const void* x, const float* signs, void* codes, float* scales, int B,
                          int H, int N, int d, void* stream) {
  return fa_fp8_quantize_ex(x, signs, codes, scales, B, H, N, d, FA_FP8_SCALE_AMAX, stream);
}

fa_status fa_fp8_quantize_ex(const void* x, const float* signs, void* codes, float* scales,
                             int B, int H, int N, int d, int scale_rule, void* stream) {
  if (scale_rule != FA_FP8_SCALE_AMAX && scale_rule != FA_FP8_SCALE_POW2)
    return fail(FA_ERR_INVALID_ARG, "scale_rule must be FA_FP8_SCALE_AMAX or FA_FP8_SCALE_POW2");
  if (!aligned16(x) || !aligned16(codes) || !scales || (reinterpret_cast<uintptr_t>(scales) & 3u))
    return fail(FA_ERR_INVALID_ARG,
                "x and codes must be non-NULL and 16-byte aligned, scales non-NULL and 4-byte aligned");
  if (signs && (reinterpret_cast<uintptr_t>(signs) & 3u))
    return fail(FA_ERR_INVALID_ARG, "signs must be 4-byte aligned");
  if (B < 1 || H < 1 || N < 1) return fail(FA_ERR_INVALID_ARG, "B, H and N must be >= 1");
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "quantisation supports d = 64 or 128");
  if ((long long)B * H * ((N + 63) / 64) > 0x7FFFFFFFLL)
    return fail(FA_ERR_INVALID_ARG, "problem too large for one launch");
  fa::QuantArgs a{};
  a.x = x; a.signs = signs; a.codes = codes; a.scales = scales;
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.pow2 = scale_rule == FA_FP8_SCALE_POW2;
  a.stream = stream;
  hipError_t e = fa::launch_fp8_quant(a);
  if (e != hipSuccess) return hip_fail(e, "fa_fp8_quantize launch");
  g_last_error.clear();
  return FA_OK;
}

// Two fp32 row arrays, -D and -LSE/scale, the second starting 256-byte
// aligned after the first.
static size_t bwd_rows_padded(size_t rows) { return (rows + 63u) & ~(size_t)63u; }

size_t fa_bwd_workspace_bytes(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1) return 0;
  const size_t rows = (size_t)B * H * (size_t)N;
  const size_t n = (bwd_rows_padded(rows) + rows) * 4u;
  return (n + 255u) & ~(size_t)255u;
}

fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                    float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (dtype != FA_BF16 && dtype != FA_FP16)
    return fail(FA_ERR_INVALID_ARG, "dtype must be FA_BF16 or FA_FP16");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(FA_ERR_INVALID_ARG,
                "q, k, v, o, dout, lse, dq, dk and dv must be non-NULL and 16-byte aligned");
  if (B < 1 || H < 1 || N < 1) return fail(FA_ERR_INVALID_ARG, "B, H and N must be >= 1");
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1");
  if (!good_scale(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if ((long long)B * H * ((N + 31) / 32) > 0x7FFFFFFFLL)
    return fail(FA_ERR_INVALID_ARG, "problem too large for one launch");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "backward supports d = 64 or 128");
  if ((long long)N * d * 2 >= (1LL << 32))
    return fail(FA_ERR_UNSUPPORTED, "one (batch, head) slice must be smaller than 4 GiB");
  const size_t need = fa_bwd_workspace_bytes(B, H, N);
  void* ws = workspace;
  std::unique_lock<std::mutex> ws_lock;   // held through the launch when ws is library-owned
  if (!workspace) {
    if (workspace_bytes != 0) return fail(FA_ERR_WORKSPACE, "workspace is NULL but workspace_bytes is not 0");
    fa_status st = owned_workspace(need, &ws, ws_lock);
    if (st != FA_OK) return st;
  } else {
    if (!aligned16(workspace)) return fail(FA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    if (workspace_bytes < need) return fail(FA_ERR_WORKSPACE, "workspace smaller than fa_bwd_workspace_bytes()");
  }
  fa::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.ndsum = static_cast<float*>(ws);
  a.nlse = a.ndsum + bwd_rows_padded((size_t)B * H * (size_t)N);
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * kLog2e);
  a.causal = causal ? 1 : 0;
  a.in_f16 = dtype == FA_FP16;
  a.stream = stream;
  hipError_t e = fa::launch_bwd(a);
  if (e != hipSuccess) return hip_fail(e, "fa_bwd launch");
  g_last_error.clear();
  return FA_OK;
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                 float scale, int causal, void* workspace, size_t workspace_bytes, void* stream) {
  return fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, FA_BF16, workspace,
                   workspace_bytes, stream);
}

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                        int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int d,
                        float scale, int causal, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(FA_ERR_INVALID_ARG,
                "q, k, v, o, dout, lse, dq, dk and dv must be non-NULL and 16-byte aligned");
  if (!cu_seqlens_q || !cu_seqlens_k ||
      ((reinterpret_cast<uintptr_t>(cu_seqlens_q) | reinterpret_cast<uintptr_t>(cu_seqlens_k)) & 3u))
    return fail(FA_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must be non-NULL and 4-byte aligned");
  if (B < 1 || H < 1) return fail(FA_ERR_INVALID_ARG, "B and H must be >= 1");
  if (max_seqlen_q < 1 || max_seqlen_k < 1 || total_q < 1 || total_k < 1)
    return fail(FA_ERR_INVALID_ARG, "max_seqlen_q, max_seqlen_k, total_q and total_k must be >= 1");
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1");
  if (!good_scale(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "varlen backward supports d = 64 or 128");
  const int longest = max_seqlen_q > max_seqlen_k ? max_seqlen_q : max_seqlen_k;
  if ((long long)B * H * ((longest + 31) / 32) > 0x7FFFFFFFLL ||
      (long long)total_q * H > 0x7FFFFFFFLL)
    return fail(FA_ERR_INVALID_ARG, "problem too large for one launch");
  // one sequence of one head is addressed with 32-bit byte offsets over its rows
  const long long row_bytes = (long long)H * d * 2;
  if ((long long)max_seqlen_q * row_bytes >= (1LL << 32) || (long long)max_seqlen_k * row_bytes >= (1LL << 32))
    return fail(FA_ERR_UNSUPPORTED, "one sequence must span under 4 GiB of rows");
  // D (fp32 [H, total_q]) takes the dense workspace of one (batch) of total_q rows
  const size_t need = fa_bwd_workspace_bytes(1, H, total_q);
  void* ws = workspace;
  std::unique_lock<std::mutex> ws_lock;   // held through the launch when ws is library-owned
  if (!workspace) {
    if (workspace_bytes != 0) return fail(FA_ERR_WORKSPACE, "workspace is NULL but workspace_bytes is not 0");
    fa_status st = owned_workspace(need, &ws, ws_lock);
    if (st != FA_OK) return st;
  } else {
    if (!aligned16(workspace)) return fail(FA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE, "workspace smaller than fa_bwd_workspace_bytes(1, H, total_q)");
  }
  fa::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.ndsum = static_cast<float*>(ws);
  a.nlse = a.ndsum + bwd_rows_padded((size_t)H * total_q);
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.B = B; a.H = H; a.N = max_seqlen_q; a.d = d;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * kLog2e);
  a.causal = causal ? 1 : 0;
  a.in_f16 = 0;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.Nk = max_seqlen_k;
  a.total_q = total_q;
  a.total_k = total_k;
  a.stream = stream;
  hipError_t e = fa::launch_bwd(a);
  if (e != hipSuccess) return hip_fail(e, "fa_bwd_varlen launch");
  g_last_error.clear();
  return FA_OK;
}

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
  }
  return "FA_UNKNOWN_STATUS";
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
