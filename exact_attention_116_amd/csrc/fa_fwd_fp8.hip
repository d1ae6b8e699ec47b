// FlashAttention forward pass with block-scaled fp8 (OCP E4M3FN) inputs on
// the gfx950 matrix cores.
//
// Method: the tiled forward pass with the running max and running sum of the
// "Flash Attention" Markdown note ("Tiling（分块）技术", "递归计算softmax"), with
// Q, K and V held as 8-bit floats plus one fp32 scale per 64 consecutive
// sequence rows of each (batch, head) -- the block quantisation of the
// FlashAttention-3 snippets.  The real value of an element is code * scale.
//
// gfx950 mapping (shared with the bf16 kernel: one wave per 32 queries, the
// transposed score tile S^T = K Q^T so that each lane owns one query)
//  * Both products run on the 32x32x64 fp8 MFMA (unscaled form): S^T from
//    K codes (LDS, A operand) and Q codes (VGPRs, B operand); O^T += V^T P^T
//    from V codes (LDS, transposed) and P rounded to E4M3FN (B operand).
//  * A key tile is 64 keys, exactly one scale block of K and of V, and the 32
//    queries of a wave lie in one scale block of Q.  So the score scale is
//    scale * log2(e) * s_q * s_k, one scalar per lane and tile, folded into
//    the FMA that feeds exp2.
//  * V's block scale is folded into P before it is rounded: the weights of
//    tile t are multiplied by sigma_t = 256 * s_v(t) / max_t s_v(t) (added
//    to the exp2 argument as log2 sigma_t), and the row sum accumulates
//    the weights divided by sigma_t.  The accumulator then holds
//    (256 / max s_v) * sum_j p_j v_j, undone once in the epilogue.
//  * The running max is moved only when it would grow by more than 0.75 (base
//    2), so every weight times sigma_t stays below 256 * 2^0.75 < 448, the
//    largest E4M3FN value; skipped rescales leave the result exact.
//  * K/V/Q codes are read through buffer resources over the head, so tile
//    rows past N read as 0 with no per-load branch.
//  * The contraction order over d (for S) and over keys (for P*V) is a
//    bijection chosen so that each lane reads 32 contiguous bytes; A and B
//    operands of one product always use the same order, so the products are
//    the full dot products whatever order the MFMA uses internally.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

namespace {
constexpr int D = 128;
constexpr int BC = 64;          // keys per tile: one scale block of K and V
constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr int BR = NW * 32;     // queries per workgroup
constexpr int KST = D + 16;     // bytes per K row in LDS
constexpr int VST = BC + 16;    // bytes per V^T row in LDS
constexpr int KTILE = BC * KST;
constexpr int VTILE = D * VST;
constexpr float kPScale = 256.f;
constexpr float kLazy = 0.75f;  // 256 * 2^0.75 = 430.5 < 448
}  // namespace

__device__ __forceinline__ f32x16 mfma32x32x64_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// Pack four floats to E4M3FN bytes (x0 in the lowest byte).
__device__ __forceinline__ uint32_t pack_fp8x4(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return (uint32_t)w;
}

template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT)))
__attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_fp8_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                       const uint8_t* __restrict__ v, const float* __restrict__ qs,
                       const float* __restrict__ ks, const float* __restrict__ vs,
                       bf16* __restrict__ o, float* __restrict__ lse, int BH, int N,
                       float c /* scale*log2(e) */) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (KTILE + VTILE)];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  const int nqt = (N + BR - 1) / BR;
  const int nsb = (N + 63) / 64;   // scale blocks per (b, h)
  const int bh = blockIdx.x % BH;
  int qt = blockIdx.x / BH;
  if constexpr (CAUSAL) qt = nqt - 1 - qt;  // longest query tiles first
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint8_t* Qh = q + head;
  const uint8_t* Kh = k + head;
  const uint8_t* Vh = v + head;
  const float* qsh = qs + (size_t)bh * nsb;
  const float* ksh = ks + (size_t)bh * nsb;
  const float* vsh = vs + (size_t)bh * nsb;

  // largest V block scale of this head (sets the pre-scale of P)
  float svmax = 0.f;
  for (int i = lane; i < nsb; i += 64) svmax = fmaxf(svmax, vsh[i]);
  svmax = wave_max(svmax);

  const int q0 = qt * BR;
  const int qw = q0 + wave * 32;
  const int my_q = qw + l32;
  const float sq = (qw < N) ? qsh[qw >> 6] : 1.f;

  // Q, K and V codes of this head through buffer resources: rows past N read 0
  const uint32_t head_bytes = (uint32_t)N * D;
  const rsrc_t Qr = make_rsrc(Qh, head_bytes);
  const rsrc_t Kr = make_rsrc(Kh, head_bytes);
  const rsrc_t Vr = make_rsrc(Vh, head_bytes);

  // Q codes as the B operand: lane (query my_q, half g), step u holds
  // d = 64u + 32g .. 64u + 32g + 31.
  i32x8 qb[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t off = (uint32_t)my_q * D + 64 * u + 32 * g;
    const u32x4 lo = buf_load16(Qr, off), hi = buf_load16(Qr, off + 16);
    qb[u] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kv_end + BC - 1) / BC;

  // ---- global -> register staging of one K/V tile ----
  // K: 64 rows x 128 B = 512 chunks of 16 B, KIT per thread.  V: 256 units
  // of 4 keys x 8 d, one for each of the first 256 threads (whole waves).
  constexpr int KIT = BC * D / 16 / NT;
  static_assert(KIT * NT == BC * D / 16 && (BC / 4) * (D / 8) == 256 && NT >= 256, "tile staging");
  const uint32_t k_off = (uint32_t)tid * 16u;
  const int kg = tid & 15, dc = (tid >> 4) & 15;
  const uint32_t v_off = (uint32_t)(4 * kg * D + 8 * dc);
  const bool v_unit = tid < 256;
  u32x4 kreg[KIT];
  u32x2 vreg[4];
  auto load_tile = [&](int j) {
    const uint32_t tile = (uint32_t)j * BC * D;
#pragma unroll
    for (int it = 0; it < KIT; ++it) kreg[it] = buf_load16(Kr, tile + k_off + it * NT * 16);
    if (v_unit) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vreg[r] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(Vr, tile + v_off + r * D, 0, 0));
    }
  };
  // V^T row d holds the tile's 64 keys as 16 groups of 4; group kg sits at
  // dword (kg & 1) * 8 + kg / 2, so lane half g finds its groups g, g+2, ..
  // g+14 -- the keys its P^T operand holds, in the same order -- in 32
  // contiguous bytes.
  auto store_tile = [&](int buf) {
    uint8_t* Ks = smem + buf * (KTILE + VTILE);
    uint8_t* Vs = Ks + KTILE;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int ch = it * NT + tid;
      *reinterpret_cast<u32x4*>(Ks + (ch >> 3) * KST + (ch & 7) * 16) = kreg[it];
    }
    if (v_unit) {
      const int pos = ((kg & 1) * 8 + (kg >> 1)) * 4;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t a = vreg[0][w], b = vreg[1][w], cc = vreg[2][w], dd = vreg[3][w];
        const uint32_t ab_lo = __builtin_amdgcn_perm(b, a, 0x05010400u);    // a0 b0 a1 b1
        const uint32_t ab_hi = __builtin_amdgcn_perm(b, a, 0x07030602u);    // a2 b2 a3 b3
        const uint32_t cd_lo = __builtin_amdgcn_perm(dd, cc, 0x05010400u);  // c0 d0 c1 d1
        const uint32_t cd_hi = __builtin_amdgcn_perm(dd, cc, 0x07030602u);  // c2 d2 c3 d3
        const uint32_t col[4] = {
            __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u),   // keys 0..3 of d = 8dc + 4w
            __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u),   // d + 1
            __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u),   // d + 2
            __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u)};  // d + 3
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<uint32_t*>(Vs + (8 * dc + 4 * w + e) * VST + pos) = col[e];
      }
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};
  float m = kNegInf;   // reference max (base 2, true scores)
  float l = 0.f;       // this lane's share of the row sum

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
      const uint8_t* Ks = smem + buf * (KTILE + VTILE);
      const uint8_t* Vs = Ks + KTILE;

      // ---- S^T = K Q^T on codes ----
      f32x16 s[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        s[b] = f32x16{};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4* src = reinterpret_cast<const u32x4*>(Ks + (32 * b + l32) * KST + 64 * u + 32 * g);
          const u32x4 lo = src[0], hi = src[1];
          const i32x8 ka = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          s[b] = mfma32x32x64_fp8(ka, qb[u], s[b]);
        }
      }

      const bool edge = (CAUSAL && kb + BC - 1 > qw) || kb + BC > N;
      if (edge) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb + 32 * b + 8 * (i >> 2) + 4 * g + (i & 3);
            const bool dead = key >= N || (CAUSAL && key > my_q);
            s[b][i] = dead ? kNegInf : s[b][i];
          }
      }

      // ---- online softmax (base 2) with the block scales folded in ----
      const float svt = vsh[j];
      const float ce = c * sq * ksh[j];
      float mx = kNegInf;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[b][i]);
      mx = max_pair32(mx) * ce;
      const float m_cand = fmaxf(m, mx);
      if (__builtin_amdgcn_ballot_w64(m_cand > m + kLazy)) {
        const float alpha = (m_cand == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m - m_cand);
        m = m_cand;
        l *= alpha;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[cb][i] *= alpha;
      }
      const float mref = (m == kNegInf) ? 0.f : m;
      const float lsig = __builtin_amdgcn_logf(kPScale * (svt / svmax));   // log2 sigma_t
      const float bias = lsig - mref;

      float p[2][16];
      float tsum = 0.f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[b][i] = __builtin_amdgcn_exp2f(fmaf(s[b][i], ce, bias));
          tsum += p[b][i];
        }
      l = fmaf(tsum, __builtin_amdgcn_exp2f(-lsig), l);

      // P^T as the B operand: dword t holds keys 8t + 4g + 0..3 of the tile
      i32x8 pb;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int b = t >> 2, i0 = 4 * (t & 3);
        pb[t] = (int)pack_fp8x4(p[b][i0], p[b][i0 + 1], p[b][i0 + 2], p[b][i0 + 3]);
      }

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const u32x4* src = reinterpret_cast<const u32x4*>(Vs + (32 * cb + l32) * VST + 32 * g);
        const u32x4 lo = src[0], hi = src[1];
        const i32x8 va = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        acc[cb] = mfma32x32x64_fp8(va, pb, acc[cb]);
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc * (max s_v / 256) / l, LSE = (m + log2 l) ln 2 ----
  l = sum_pair32(l);
  const float fac = (svmax / kPScale) / l;
  if (my_q < N) {
    const size_t row = (size_t)bh * N + my_q;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int d0 = 32 * cb + 8 * ii + 4 * g;
        const float o0 = acc[cb][4 * ii] * fac, o1 = acc[cb][4 * ii + 1] * fac;
        const float o2 = acc[cb][4 * ii + 2] * fac, o3 = acc[cb][4 * ii + 3] * fac;
        *reinterpret_cast<u32x2*>(o + row * D + d0) = u32x2{pack_bf16(o0, o1), pack_bf16(o2, o3)};
      }
    if (g == 0) lse[row] = (m + __builtin_amdgcn_logf(l)) * kLn2;
  }
}

hipError_t launch_fwd_fp8(const FwdArgs& a) {
  if (a.d != D || a.out_f32) return hipErrorNotSupported;
  const int nqt = (a.N + BR - 1) / BR;
  const long long blocks = (long long)nqt * a.B * a.H;
  const int BH = a.B * a.H;
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NT), 0, (hipStream_t)a.stream,
                       (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, a.q_scale,
                       a.k_scale, a.v_scale, (bf16*)a.o, a.lse, BH, a.N, a.scale_log2);
  };
  if (a.causal)
    args(fa_fwd_fp8_kernel<true>);
  else
    args(fa_fwd_fp8_kernel<false>);
  return hipGetLastError();
}

}  // namespace fa
