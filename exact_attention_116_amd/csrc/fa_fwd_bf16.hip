// FlashAttention forward pass, bf16 inputs, on gfx950 matrix cores.
//
// Method (the "Flash Attention" Markdown note, sections "Tiling（分块）技术"
// and "递归计算softmax"; loop order from the FlashAttention-2 overview):
// queries are tiled in the outer loop (one workgroup per query tile of one
// (batch, head)), keys/values in the inner loop.  For every key tile the
// kernel forms the scores, updates a running row max m and row sum l,
// rescales the output accumulator by exp(m_old - m_new) and adds P*V.  The
// N x N scores never leave registers.  The output is divided by l once at
// the end and the log-sum-exp m + ln l is stored for each query.
//
// gfx950 mapping
//  * Each wave owns 32 queries (FA-2's split of the query rows over warps:
//    no softmax state is shared between waves).  It computes the
//    transposed score tile S^T = K * Q^T with the 32x32x16 bf16 MFMA, so
//    that every lane holds scores of a single query (lane%32): the row max
//    and row sum are in-lane plus one exchange between the two wave halves.
//  * Q^T is the MFMA B operand and stays in VGPRs for the whole key loop.
//  * P^T, rounded to bf16, is used directly as the B operand of
//    O^T = V^T * P^T; the output accumulator O^T again has one query per
//    lane, so the per-query rescale is a per-lane scalar.
//  * A workgroup is 8 waves (256 queries, two waves per SIMD) sharing each
//    K/V tile.  K tiles are stored row-major in LDS; V tiles are stored
//    transposed (V^T, d-major) with the keys permuted to match the order in
//    which the score accumulator hands P^T to the next MFMA.  Both are
//    double-buffered: the global loads of tile j+1 are in flight while tile
//    j is computed.  Loads go through buffer resources over the head, so
//    tile rows past N read as 0 with no branch and no 64-bit address math.
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA.  The
//    reference max is only moved (and O, l rescaled) when some lane's max
//    grows by more than 2^8; otherwise the stale reference is kept, which
//    leaves the result exact and skips most rescales.  l sums the fp32
//    probabilities (before their bf16 rounding for the MFMA), so the stored
//    log-sum-exp carries no bf16 error even for rows with few keys.
//  * Causal: key tiles entirely above the diagonal are never loaded; within
//    a workgroup, a wave whose 32 queries all precede a tile skips its math;
//    masking is applied only on tiles that straddle the diagonal or N.
//    Query tiles are launched heaviest first.  Consecutive workgroups take
//    different heads, so with B*H a multiple of 8 every query tile of a
//    head lands on the same XCD (dispatch is round-robin over the 8 XCDs)
//    and shares its K/V in that XCD's L2.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

template <int D, int BC, int NW>
struct FwdCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BR = NW * 32;       // queries per workgroup
  static constexpr int KST = D + 8;        // K row stride in LDS (bf16 elements)
  static constexpr int VST = BC + 8;       // V^T row stride in LDS
  static constexpr int KTILE = BC * KST;
  static constexpr int VTILE = D * VST;
  static constexpr int KCH = BC * D / 8;           // 16-byte chunks per K tile
  static constexpr int KIT = (KCH + NT - 1) / NT;  // chunks per thread
  static constexpr int VU = (BC / 4) * (D / 8);    // (4 keys x 8 d) units per V tile
    static_assert(BC % 32 == 0 && D % 32 == 0, "tile shapes");
};

// Position (in 4-key groups) of key group kg inside a V^T row.  Within each
// 32-key block the score accumulator of lane half h holds key groups
// {h, h+2} for the first 16-key MFMA step and {4+h, 6+h} for the second;
// swapping bits 0 and 1 of the group index makes each of those a
// contiguous 8-key run, readable with one 16-byte LDS load.
__device__ __forceinline__ int vt_group_pos(int kg) {
  const int g = kg & 7;
  return (kg & ~7) | (g & 4) | ((g & 1) << 1) | ((g >> 1) & 1);
}

template <int D, int BC, int NW, bool CAUSAL, bool OUT_F32>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
__attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                        const bf16* __restrict__ v, void* __restrict__ o,
                        float* __restrict__ lse, int BH, int N, float c /* scale*log2(e) */) {
  using C = FwdCfg<D, BC, NW>;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (C::KTILE + C::VTILE)];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  const int nqt = (N + C::BR - 1) / C::BR;
  const int bh = blockIdx.x % BH;
  int qt = blockIdx.x / BH;
  if constexpr (CAUSAL) qt = nqt - 1 - qt;  // longest query tiles first
  const size_t head = (size_t)bh * (size_t)N * D;
  const bf16* Qh = q + head;
  const bf16* Kh = k + head;
  const bf16* Vh = v + head;

  const int q0 = qt * C::BR;
  const int qw = q0 + wave * 32;   // first query of this wave
  const int my_q = qw + l32;       // the query this lane's columns belong to

  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const rsrc_t Qr = make_rsrc(Qh, head_bytes);
  const rsrc_t Kr = make_rsrc(Kh, head_bytes);
  const rsrc_t Vr = make_rsrc(Vh, head_bytes);
  bf16x8 qb[D / 16];
#pragma unroll
  for (int u = 0; u < D / 16; ++u)
    qb[u] = __builtin_bit_cast(bf16x8, buf_load16(Qr, ((uint32_t)my_q * D + 16 * u + 8 * g) * 2u));

  const int kv_end = CAUSAL ? min(N, q0 + C::BR) : N;
  const int ntiles = (kv_end + BC - 1) / BC;

  static_assert(C::KCH % C::NT == 0 && C::VU % 64 == 0, "tile shapes");
  const uint32_t k_off = (uint32_t)tid * 16u;
  const int v_kg = tid % (BC / 4), v_dc = tid / (BC / 4);
  const uint32_t v_off = (uint32_t)(4 * v_kg * D + 8 * v_dc) * 2u;
  const bool v_unit = tid < C::VU;
  u32x4 kreg[C::KIT];
  u32x4 vreg[4];
  auto load_tile = [&](int j) {
    const uint32_t tile = (uint32_t)j * BC * D * 2u;
#pragma unroll
    for (int it = 0; it < C::KIT; ++it)
      kreg[it] = buf_load16(Kr, tile + k_off + (uint32_t)(it * C::NT * 16));
    if (v_unit) {
#pragma unroll
      for (int r = 0; r < 4; ++r) vreg[r] = buf_load16(Vr, tile + v_off + (uint32_t)(r * D * 2));
    }
  };
  auto store_tile = [&](int buf) {
    bf16* Ks = smem + buf * (C::KTILE + C::VTILE);
    bf16* Vs = Ks + C::KTILE;
#pragma unroll
    for (int it = 0; it < C::KIT; ++it) {
      const int ch = it * C::NT + tid;
      const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(Ks + row * C::KST + col) = kreg[it];
    }
    if (v_unit) {
      const int pos = 4 * vt_group_pos(v_kg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t p01 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);
        const uint32_t p23 = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], sel);
        *reinterpret_cast<u32x2*>(Vs + (8 * v_dc + e) * C::VST + pos) = u32x2{p01, p23};
      }
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};
  float m = kNegInf;   // reference max, base-2 units of the scaled scores
  float l = 0.f;       // this lane's share of the row sum (keys of its half)

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < ntiles;
    if (more) load_tile(j + 1);

    const int kb = j * BC;
    const bool active = !CAUSAL || kb <= qw + 31;
    if (active) {
      const bf16* Ks = smem + buf * (C::KTILE + C::VTILE);
      const bf16* Vs = Ks + C::KTILE;

      // ---- S^T = K * Q^T : keys on rows, this lane's query on the column ----
      f32x16 s[BC / 32];
#pragma unroll
      for (int b = 0; b < BC / 32; ++b) s[b] = f32x16{};
#pragma unroll
      for (int u = 0; u < D / 16; ++u) {
#pragma unroll
        for (int b = 0; b < BC / 32; ++b) {
          const bf16x8 ka =
              *reinterpret_cast<const bf16x8*>(Ks + (32 * b + l32) * C::KST + 16 * u + 8 * g);
          s[b] = mfma32x32x16(ka, qb[u], s[b]);
        }
      }

      // ---- mask keys past the diagonal or past N (edge tiles only) ----
      const bool edge = (CAUSAL && kb + BC - 1 > qw) || kb + BC > N;
      if (edge) {
#pragma unroll
        for (int b = 0; b < BC / 32; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb + 32 * b + 8 * (i >> 2) + 4 * g + (i & 3);
            const bool dead = key >= N || (CAUSAL && key > my_q);
            s[b][i] = dead ? kNegInf : s[b][i];
          }
      }

      // ---- online softmax (base 2) ----
      float mx = kNegInf;
#pragma unroll
      for (int b = 0; b < BC / 32; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[b][i]);
      mx = max_pair32(mx) * c;
      const float m_cand = fmaxf(m, mx);
      // move the reference max only when it would grow by more than 2^8
      if (__builtin_amdgcn_ballot_w64(m_cand > m + 8.f)) {
        const float alpha = (m_cand == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m - m_cand);
        m = m_cand;
        l *= alpha;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[cb][i] *= alpha;
      }
      const float mref = (m == kNegInf) ? 0.f : m;

      // P^T in bf16, grouped as the B operands of the 16-key MFMA steps
      bf16x8 pb[BC / 16];
#pragma unroll
      for (int t = 0; t < BC / 16; ++t) {
        uint32_t w[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[t >> 1][8 * (t & 1) + 2 * h], c, -mref));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[t >> 1][8 * (t & 1) + 2 * h + 1], c, -mref));
          w[h] = pack_bf16(p0, p1);
          l += p0 + p1;
        }
        pb[t] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
      }

      // ---- O^T += V^T * P^T ----
#pragma unroll
      for (int t = 0; t < BC / 16; ++t) {
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) {
          const bf16x8 va =
              *reinterpret_cast<const bf16x8*>(Vs + (32 * cb + l32) * C::VST + 16 * t + 8 * g);
          acc[cb] = mfma32x32x16(va, pb[t], acc[cb]);
        }
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2 ----
  l = sum_pair32(l);
  const float inv = 1.f / l;
  if (my_q < N) {
    const size_t row = (size_t)bh * N + my_q;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int d0 = 32 * cb + 8 * ii + 4 * g;
        const float o0 = acc[cb][4 * ii] * inv, o1 = acc[cb][4 * ii + 1] * inv;
        const float o2 = acc[cb][4 * ii + 2] * inv, o3 = acc[cb][4 * ii + 3] * inv;
        if constexpr (OUT_F32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(o) + row * D + d0) = f32x4{o0, o1, o2, o3};
        } else {
          *reinterpret_cast<u32x2*>(static_cast<bf16*>(o) + row * D + d0) =
              u32x2{pack_bf16(o0, o1), pack_bf16(o2, o3)};
        }
      }
    if (g == 0) lse[row] = (m + __builtin_amdgcn_logf(l)) * kLn2;
  }
}

template <int D, int BC, int NW, bool CAUSAL, bool OUT_F32>
static hipError_t launch(const FwdArgs& a) {
  using C = FwdCfg<D, BC, NW>;
  const int nqt = (a.N + C::BR - 1) / C::BR;
  const long long blocks = (long long)nqt * a.B * a.H;
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, BC, NW, CAUSAL, OUT_F32>), dim3((unsigned)blocks),
                     dim3(C::NT), 0, (hipStream_t)a.stream, (const bf16*)a.q, (const bf16*)a.k,
                     (const bf16*)a.v, a.o, a.lse, a.B * a.H, a.N, a.scale_log2);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool OUT_F32>
static hipError_t launch_d(const FwdArgs& a) {
  return launch<D, 64, 8, CAUSAL, OUT_F32>(a);
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  const bool c = a.causal != 0, f = a.out_f32 != 0;
  if (a.d == 128) {
    if (c) return f ? launch_d<128, true, true>(a) : launch_d<128, true, false>(a);
    return f ? launch_d<128, false, true>(a) : launch_d<128, false, false>(a);
  }
  if (c) return f ? launch_d<64, true, true>(a) : launch_d<64, true, false>(a);
  return f ? launch_d<64, false, true>(a) : launch_d<64, false, false>(a);
}

}  // namespace fa
