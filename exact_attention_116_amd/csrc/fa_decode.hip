// Split-KV single-query decode (Flash-Decoding) and the merge of its splits.
//
// Method: with one query per (batch, head) the forward pass has no query
// tiles to spread over the GPU, so the key/value cache is cut into
// num_splits ranges and each range is reduced independently to a partial
// output and its log-sum-exp (the two-part K/V split example of the
// FlashAttention-2 overview snippets, generalised; the Flash-Decoding
// snippet's parallelism over the KV length).  A second kernel merges the
// partials, weighting each by exp(LSE_s - LSE) (the splitK combine of the
// FlashAttention-3 snippets).
//
// gfx950 mapping: this is a streaming read of the whole cache, bound by
// HBM bandwidth, not by arithmetic, so it uses no MFMA.  Each thread keeps
// 16 K and 16 V rows (16 bytes each) in flight, read with the non-temporal
// cache hint since every byte is used exactly once.  d/8 lanes share one
// key row (16-byte loads, each wave instruction reads 64 x 16 B of
// consecutive rows), the dot products use v_dot2_f32_bf16 plus a DPP
// reduction inside the lane group, and every lane group keeps its own
// online-softmax state (max, sum, 8 output columns) over its keys.  Those
// states are merged through LDS at the end of the workgroup, so the key loop
// has no barriers and no cross-group traffic.
#include "fa_device.hpp"
#include "fa_internal.h"

#include <mutex>

namespace fa {

template <int D, int NW, int U>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
void fa_decode_split_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kc,
                            const bf16* __restrict__ vc, float* __restrict__ part_o,
                            float* __restrict__ part_lse, int Lkv, int S, int chunk, float c) {
  constexpr int LPR = D / 8;        // lanes per key row
  constexpr int RPW = 64 / LPR;     // key rows per wave instruction
  constexpr int NG = NW * RPW;      // lane groups in the workgroup
  constexpr int STEP = NG;          // keys per workgroup step
  __shared__ float sm_m[NG], sm_l[NG];
  __shared__ float sm_o[NG][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int dl = lane % LPR, rg = lane / LPR;
  const int grp = wave * RPW + rg;
  const int bh = blockIdx.x / S, s = blockIdx.x % S;
  const long long lo_ll = (long long)s * chunk;
  const int lo = (int)(lo_ll < Lkv ? lo_ll : Lkv);
  const int hi = (int)((long long)lo + chunk < Lkv ? (long long)lo + chunk : Lkv);

  const u32x4 qv = *reinterpret_cast<const u32x4*>(q + (size_t)bh * D + 8 * dl);
  // K/V rows of this split through buffer resources spanning exactly
  // [lo, hi): rows past hi read as 0 (and are masked below).  The cache is
  // streamed once, so the loads carry the non-temporal hint.
  const size_t head = (size_t)bh * (size_t)Lkv * D + (size_t)lo * D;
  const uint32_t span = (uint32_t)(hi - lo) * D * 2u;
  const rsrc_t Kr = make_rsrc(kc + head, span);
  const rsrc_t Vr = make_rsrc(vc + head, span);

  float m = kNegInf, l = 0.f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;

  for (int base = lo; base < hi; base += U * STEP) {
    u32x4 kr[U], vr[U];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const uint32_t off = ((uint32_t)(base - lo + uu * STEP + grp) * D + 8 * dl) * 2u;
      kr[uu] = buf_load16_nt(Kr, off);
      vr[uu] = buf_load16_nt(Vr, off);
    }
    float sc[U];
    float mx = kNegInf;
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      float d = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        d = dot2_bf16(qv[w], kr[uu][w], d);
      d = group_sum<LPR>(d) * c;
      sc[uu] = (base + uu * STEP + grp < hi) ? d : kNegInf;
      mx = fmaxf(mx, sc[uu]);
    }
    const float mnew = fmaxf(m, mx);
    const float mref = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m - mref);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const float p = __builtin_amdgcn_exp2f(sc[uu] - mref);
      l += p;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc[2 * w] = fmaf(p, bf16lo(vr[uu][w]), acc[2 * w]);
        acc[2 * w + 1] = fmaf(p, bf16hi(vr[uu][w]), acc[2 * w + 1]);
      }
    }
  }

  // merge the lane groups of the workgroup
  if (dl == 0) {
    sm_m[grp] = m;
    sm_l[grp] = l;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sm_o[grp][8 * dl + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float M = kNegInf;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) M = fmaxf(M, sm_m[gi]);
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const float w = __builtin_amdgcn_exp2f(sm_m[gi] - M);  // -inf -> 0
        L = fmaf(w, sm_l[gi], L);
        O = fmaf(w, sm_o[gi][tid], O);
      }
    }
    const size_t ps = (size_t)bh * S + s;
    part_o[ps * D + tid] = (M == kNegInf) ? 0.f : O / L;
    if (tid == 0) part_lse[ps] = (M == kNegInf) ? kNegInf : (M + __builtin_amdgcn_logf(L)) * kLn2;
  }
}

// O = sum_s w_s O_s / sum_s w_s with w_s = exp(LSE_s - max_s LSE_s).
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(D, D)))
void fa_decode_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                              bf16* __restrict__ o, float* __restrict__ lse, int S) {
  constexpr float kLog2e = 1.44269504088896340736f;
  const int bh = blockIdx.x, t = threadIdx.x;
  const float* pl = part_lse + (size_t)bh * S;
  const float* po = part_o + (size_t)bh * S * D + t;
  // (unrolled so that many independent loads are in flight: the loop is
  // latency-bound, not bandwidth-bound)
  float M = kNegInf;
#pragma unroll 16
  for (int s = 0; s < S; ++s) M = fmaxf(M, pl[s]);
  float W = 0.f, O = 0.f;
  if (M != kNegInf) {
#pragma unroll 16
    for (int s = 0; s < S; ++s) {
      const float w = __builtin_amdgcn_exp2f((pl[s] - M) * kLog2e);
      W += w;
      O = fmaf(w, po[(size_t)s * D], O);
    }
  }
  const float out = (M == kNegInf) ? 0.f : O / W;
  o[(size_t)bh * D + t] = (bf16)out;
  if (lse && t == 0) lse[bh] = (M == kNegInf) ? kNegInf : M + __builtin_amdgcn_logf(W) * kLn2;
}

template <int D>
static hipError_t launch_d(const DecodeArgs& a) {
  constexpr int NW = 4, U = 16;
  const int BH = a.B * a.H;
  const int chunk = (int)(((long long)a.Lkv + a.num_splits - 1) / a.num_splits);
  hipStream_t st = (hipStream_t)a.stream;
  hipLaunchKernelGGL((fa_decode_split_kernel<D, NW, U>), dim3((unsigned)((long long)BH * a.num_splits)),
                     dim3(NW * 64), 0, st, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
                     a.part_o, a.part_lse, a.Lkv, a.num_splits, chunk, a.scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine(a);
}

hipError_t launch_decode(const DecodeArgs& a) {
  return a.d == 128 ? launch_d<128>(a) : launch_d<64>(a);
}

// ---------------------------------------------------------------------------
// Fixed scratch for the decode entry point that allocates nothing: the split
// partials live in this file-scope device array (one copy per GPU, held until
// the process ends) instead of a workspace.  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address is taken
// once per device with hipGetSymbolAddress (with that device current) and
// only that address is handed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch`, per device
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_combine(const DecodeArgs& a) {
  const unsigned BH = (unsigned)(a.B * a.H);
  hipStream_t st = (hipStream_t)a.stream;
  if (a.d == 128)
    hipLaunchKernelGGL((fa_decode_combine_kernel<128>), dim3(BH), dim3(128), 0, st, a.part_o,
                       a.part_lse, (bf16*)a.o, a.lse, a.num_splits);
  else
    hipLaunchKernelGGL((fa_decode_combine_kernel<64>), dim3(BH), dim3(64), 0, st, a.part_o,
                       a.part_lse, (bf16*)a.o, a.lse, a.num_splits);
  return hipGetLastError();
}

}  // namespace fa
