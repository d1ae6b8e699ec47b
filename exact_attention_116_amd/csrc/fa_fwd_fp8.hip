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
//  * Both products run on the 32x32x64 fp8 MFMA: S^T from K codes (LDS, A
//    operand) and Q codes (VGPRs, B operand); O^T += V^T P^T from V codes
//    (LDS, read transposed, with a power-of-two block scale) and P rounded
//    to E4M3FN (B operand).
//  * A key tile is 128 keys, two scale blocks of K and of V, and the 32
//    queries of a wave lie in one scale block of Q.  So the score scale is
//    scale * log2(e) * s_q * s_k, one scalar per lane and half tile, folded
//    into the FMA that feeds exp2.
//  * P is pre-scaled by the constant 256 = 2^8 before it is rounded to
//    E4M3FN, so the largest weight of a row (exactly 1 whenever the running
//    max has just moved) stays exact.  A pre-scale that varied per V block
//    would round that weight by up to 2^-4 in every row dominated by one key.
//  * V's block scale enters outside the rounding of P.  Write s_v(t) = 2^e_t
//    * r_t with r_t in [0.5, 1).  The power of two 2^(e_t - e_max) is the
//    E8M0 scale of the V operand of the scaled fp8 MFMA (each 32x32x64
//    product covers exactly one 64-key V block), and the accumulator is kept
//    in units of the current block's r_t: before the products of block t it
//    is multiplied by r_{t-1} / r_t (merged with the running-max rescale).
//    The epilogue multiplies by r_last * 2^e_max once.  When every V scale
//    of the head has the same mantissa (power-of-two scales, say), all the
//    ratios are 1 and the loop runs in a second form without those
//    multiplies: one multiply per accumulator element and 64 keys fewer.
//  * The running max is moved only when it would grow by more than 0.75 (base
//    2), so every weight times 256 stays below 256 * 2^0.75 < 448, the
//    largest E4M3FN value; skipped rescales leave the result exact.
//  * K and V tiles go from HBM straight to LDS with direct buffer loads (rows
//    past N read as 0 through the buffer range), double-buffered, the loads
//    of tile j+1 issued while tile j is computed.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

namespace {
template <bool B> struct BoolC { static constexpr bool value = B; };
constexpr int D = 128;
constexpr float kLog2PScale = 8.f;  // P is rounded as 256 * p
constexpr float kLazy = 0.75f;      // 256 * 2^0.75 = 430.5 < 448
constexpr int kE8M0One = 127;       // E8M0 code of 2^0
}  // namespace

__device__ __forceinline__ f32x16 mfma32x32x64_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same product with the A operand multiplied by 2^(sa - 127): sa is an
// E8M0 code (the same in every lane here, so it scales all of A); B is
// unscaled (code 127).
__device__ __forceinline__ f32x16 mfma32x32x64_fp8_sa(const i32x8& a, const i32x8& b, const f32x16& c,
                                                      int sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, kE8M0One);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// Pack four floats to E4M3FN bytes (x0 in the lowest byte).  The first
// conversion's other half is overwritten by the second, so it starts from
// x0's own bits rather than a zeroed register (no v_mov per word).
__device__ __forceinline__ uint32_t pack_fp8x4(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, __builtin_bit_cast(int, x0), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return (uint32_t)w;
}

// ---------------------------------------------------------------------------
// V^T operands come from ds_read_b64_tr_b8: within
// each 16-lane group, lane i receives byte i%8 of the 8-byte pieces
// addressed by lanes i/8, i/8 + 2, .., i/8 + 14, so when lanes 2e and 2e+1
// point at the same key row, 8 columns apart, one read hands every lane
// eight keys of its own column (16 columns per group).  Four reads fill the
// 32 key slots of the 32x32x64 A operand in the order the score accumulator
// hands P^T over.  16-byte chunks are XOR-swizzled by row: K by (r/2)%8 so
// that row-wise reads of 16 consecutive rows hit distinct banks, V by
// 2*((r/2)%2) + 4*((r/8)%2) so that the eight rows of a transposing read do.
// ---------------------------------------------------------------------------
namespace {
constexpr int BC2 = 128;        // keys per tile: two scale blocks
constexpr int RB8 = D;          // bytes per fp8 row
__device__ __forceinline__ int swz_k8(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_v8(int r) { return 2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1); }
typedef int i32x2 __attribute__((ext_vector_type(2)));
}  // namespace

template <bool CAUSAL, int NW2>
__global__ __attribute__((amdgpu_flat_work_group_size(NW2 * 64, NW2 * 64)))
__attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_fp8_dl_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                          const uint8_t* __restrict__ v, const float* __restrict__ qs,
                          const float* __restrict__ ks, const float* __restrict__ vs,
                          bf16* __restrict__ o, float* __restrict__ lse, int BH, int N,
                          float c /* scale*log2(e) */) {
  constexpr int BRW = NW2 * 32;               // queries per workgroup
  constexpr int TB = BC2 * RB8;               // bytes of one K (or V) tile
  constexpr int NI = TB / 1024;               // 1 KB direct loads per tile and tensor
  constexpr int IPW = NI / NW2;
  static_assert(NI % NW2 == 0, "tile loads split evenly over the waves");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS targets in SGPRs
  const int l32 = lane & 31, g = lane >> 5;

  const int nqt = (N + BRW - 1) / BRW;
  const int nsb = (N + 63) / 64;
  const int bh = blockIdx.x % BH;
  int qt = blockIdx.x / BH;
  if constexpr (CAUSAL) qt = nqt - 1 - qt;  // longest query tiles first
  const size_t head = (size_t)bh * (size_t)N * D;
  const float* qsh = qs + (size_t)bh * nsb;
  const float* ksh = ks + (size_t)bh * nsb;
  const float* vsh = vs + (size_t)bh * nsb;

  // the binary exponent of the head's largest V scale: every block's
  // power of two is taken relative to it (E8M0 codes <= 127)
  float svmax = 0.f;
  for (int i = lane; i < nsb; i += 64) svmax = fmaxf(svmax, vsh[i]);
  svmax = wave_max(svmax);
  const int e_max = __builtin_amdgcn_frexp_expf(svmax);
  // do all V scales of the head share one mantissa?
  const float r_first = __builtin_amdgcn_frexp_mantf(vsh[0]);
  bool rdiff = false;
  for (int i = lane; i < nsb; i += 64) rdiff |= __builtin_amdgcn_frexp_mantf(vsh[i]) != r_first;
  const bool one_mantissa = __builtin_amdgcn_ballot_w64(rdiff) == 0;

  const int q0 = qt * BRW;
  const int qw = q0 + wave * 32;
  const int my_q = qw + l32;
  const float sq = (qw < N) ? qsh[qw >> 6] : 1.f;

  const uint32_t head_bytes = (uint32_t)N * D;
  const rsrc_t Qr = make_rsrc(q + head, head_bytes);
  [[maybe_unused]] const rsrc_t Kr = make_rsrc(k + head, head_bytes);
  [[maybe_unused]] const rsrc_t Vr = make_rsrc(v + head, head_bytes);

  // Q codes as the B operand: step u holds d = 64u + 32g .. +31
  i32x8 qb[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t off = (uint32_t)my_q * D + 64 * u + 32 * g;
    const u32x4 lo = buf_load16(Qr, off), hi = buf_load16(Qr, off + 16);
    qb[u] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }

  const int kv_end = CAUSAL ? min(N, q0 + BRW) : N;
  const int ntiles = (kv_end + BC2 - 1) / BC2;

  // direct loads: lane -> 16 bytes of LDS at blk*1024 + 16*lane, row r,
  // physical chunk p, fetched from logical chunk p ^ swz(r)
  uint32_t gk[IPW], gv[IPW];
#pragma unroll
  for (int x = 0; x < IPW; ++x) {
    const int byte = (wave * IPW + x) * 1024 + lane * 16;
    const int r = byte / RB8, p = (byte % RB8) / 16;
    gk[x] = (uint32_t)(r * RB8 + 16 * (p ^ swz_k8(r)));
    gv[x] = (uint32_t)(r * RB8 + 16 * (p ^ swz_v8(r)));
  }
  auto load_tile = [&](int j) {
    [[maybe_unused]] const uint32_t tile = (uint32_t)j * TB;
    [[maybe_unused]] uint8_t* Kd = smem + (j & 1) * 2 * TB;
    [[maybe_unused]] uint8_t* Vd = Kd + TB;
#if defined(__HIP_DEVICE_COMPILE__)  // the LDS-DMA builtin exists in the device pass only
#pragma unroll
    for (int x = 0; x < IPW; ++x) {
      const int blk = wave * IPW + x;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Kr, (__attribute__((address_space(3))) void*)(Kd + blk * 1024), 16, tile + gk[x], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Vr, (__attribute__((address_space(3))) void*)(Vd + blk * 1024), 16, tile + gv[x], 0, 0, 0);
    }
#endif
  };

  // LDS read offsets.  K fragment (block b, step u): row 32b + l32, logical
  // chunks 4u + 2g and 4u + 2g + 1.  V^T fragment (half h, column block cb,
  // read R): key row 64h + 16R + 8(e/4) + 4g + e%4 for source pair e =
  // (lane%16)/2, column 32cb + 16((lane/16)%2) + 8(lane%2).
  uint32_t k_rd[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      k_rd[u][hh] = (uint32_t)(l32 * RB8 + 16 * ((4 * u + 2 * g + hh) ^ swz_k8(l32)));
  uint32_t v_rd[4][D / 32];   // [R][cb], relative to the half's first row
  {
    const int s16 = lane & 15, e = s16 >> 1, odd = s16 & 1, qq = (lane >> 4) & 1;
#pragma unroll
    for (int R = 0; R < 4; ++R)
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const int r = 16 * R + 8 * (e >> 2) + 4 * g + (e & 3);
        const int ch = 2 * cb + qq;
        v_rd[R][cb] = (uint32_t)(r * RB8 + 16 * (ch ^ swz_v8(r)) + 8 * odd);
      }
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};
  float m = kNegInf;
  float l = 0.f;                                    // row sum of 256 * p
  float r_cur = __builtin_amdgcn_frexp_mantf(vsh[0]);  // units of acc

  load_tile(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  // the key loop; MULV: V's block mantissas differ, so acc changes units
  auto key_loop = [&](auto mulv) __attribute__((always_inline)) {
  constexpr bool MULV = decltype(mulv)::value;
  for (int j = 0; j < ntiles; ++j) {
    const bool more = j + 1 < ntiles;
    if (more) load_tile(j + 1);

    const int kb = j * BC2;
    const bool active = !CAUSAL || kb <= qw + 31;
    if (active) {
      const uint8_t* Ks = smem + (j & 1) * 2 * TB;
      const uint8_t* Vs = Ks + TB;

      // ---- S^T = K Q^T on codes, four 32-key blocks ----
      f32x16 s[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) s[b] = f32x16{};
      {
        constexpr int PD = 2, NF = 8;
        i32x8 kf[NF];
#pragma unroll
        for (int i = 0; i < NF + PD; ++i) {
          if (i < NF) {
            const int b = i >> 1, u = i & 1;
            const uint8_t* base = Ks + (32 * b) * RB8;
            const u32x4 lo = *reinterpret_cast<const u32x4*>(base + k_rd[u][0]);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(base + k_rd[u][1]);
            kf[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          }
          if (i >= PD) {
            const int x = i - PD, b = x >> 1, u = x & 1;
            s[b] = mfma32x32x64_fp8(kf[x], qb[u], s[b]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      const bool edge = (CAUSAL && kb + BC2 - 1 > qw) || kb + BC2 > N;
      if (edge) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb + 32 * b + 8 * (i >> 2) + 4 * g + (i & 3);
            const bool dead = key >= N || (CAUSAL && key > my_q);
            s[b][i] = dead ? kNegInf : s[b][i];
          }
      }

      // ---- online softmax, per 64-key scale block h of the tile ----
      const int sb0 = 2 * j;                       // the tile's first scale block
      const bool h1 = sb0 + 1 < nsb;               // second half exists
      const float ce0 = c * sq * ksh[sb0];
      const float ce1 = h1 ? c * sq * ksh[sb0 + 1] : ce0;
      // The row max as med3(a, b, +inf) = max(a, b): with fmaxf the compiler
      // quiets every fp8-MFMA result (v_max_f32 x, x, x) before the max, one
      // extra VALU op per score; this form compiles to v_max3 without it
      // (same results, 6% faster at B=4 H=16 N=8192).
      constexpr float kPosInf = __builtin_inff();
      float mx0 = kNegInf, mx1 = kNegInf, mx2 = kNegInf, mx3 = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        mx0 = __builtin_amdgcn_fmed3f(mx0, s[0][i], kPosInf);
        mx1 = __builtin_amdgcn_fmed3f(mx1, s[1][i], kPosInf);
        mx2 = __builtin_amdgcn_fmed3f(mx2, s[2][i], kPosInf);
        mx3 = __builtin_amdgcn_fmed3f(mx3, s[3][i], kPosInf);
      }
      mx0 = __builtin_amdgcn_fmed3f(mx0, mx1, kPosInf);
      mx1 = __builtin_amdgcn_fmed3f(mx2, mx3, kPosInf);
      float mx = fmaxf(mx0 * ce0, mx1 * ce1);
      mx = max_pair32(mx);
      const float m_cand = fmaxf(m, mx);
      float alpha = 1.f;
      if (__builtin_amdgcn_ballot_w64(m_cand > m + kLazy)) {
        alpha = (m_cand == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m - m_cand);
        m = m_cand;
        l *= alpha;
        if constexpr (!MULV) {
#pragma unroll
          for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[cb][i] *= alpha;
        }
      }
      const float mref = (m == kNegInf) ? 0.f : m;
      const float bias = kLog2PScale - mref;

      // V block t = sb0 + hh: E8M0 code of 2^(e_t - e_max) for the product,
      // and the factor that moves acc from the previous block's units r to
      // this block's (the half past N, whose keys are all masked, keeps both)
      int sa[2];
      float fac[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        if (hh == 0 || h1) {
          const float sv = vsh[sb0 + hh];
          sa[hh] = max(kE8M0One + __builtin_amdgcn_frexp_expf(sv) - e_max, 0);
          if constexpr (MULV) {
            const float rt = __builtin_amdgcn_frexp_mantf(sv);
            fac[hh] = r_cur * __builtin_amdgcn_rcpf(rt);
            r_cur = rt;
          }
        } else {
          sa[hh] = kE8M0One;
          fac[hh] = 1.f;
        }
      }
      if constexpr (MULV) {
        fac[0] *= alpha;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[cb][i] *= fac[0];
      }

      i32x8 pb[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float ce = hh == 0 ? ce0 : ce1;
        float p[2][16];
        float tsum = 0.f;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            p[bb][i] = __builtin_amdgcn_exp2f(fmaf(s[2 * hh + bb][i], ce, bias));
            tsum += p[bb][i];
          }
        l += tsum;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int bb = t >> 2, i0 = 4 * (t & 3);
          pb[hh][t] = (int)pack_fp8x4(p[bb][i0], p[bb][i0 + 1], p[bb][i0 + 2], p[bb][i0 + 3]);
        }
      }

      // ---- O^T += V^T P^T, V^T from transposing reads ----
      {
        constexpr int PD = 2, NF = 2 * (D / 32);
        i32x8 vf[NF];
#pragma unroll
        for (int i = 0; i < NF + PD; ++i) {
          if (i < NF) {
            const int hh = i / (D / 32), cb = i % (D / 32);
            const uint8_t* base = Vs + (64 * hh) * RB8;
            i32x8 f;
#pragma unroll
            for (int R = 0; R < 4; ++R) {
              const i32x2 t2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                  (__attribute__((address_space(3))) i32x2*)(base + v_rd[R][cb]));
              f[2 * R] = t2[0];
              f[2 * R + 1] = t2[1];
            }
            vf[i] = f;
          }
          if (i >= PD) {
            const int x = i - PD, hh = x / (D / 32), cb = x % (D / 32);
            // the second block's products start from acc in its units
            acc[cb] = mfma32x32x64_fp8_sa(vf[x], pb[hh], (hh == 0 || !MULV) ? acc[cb] : acc[cb] * fac[1],
                                          sa[hh]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    if (more) __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  };
  if (one_mantissa)
    key_loop(BoolC<false>{});
  else
    key_loop(BoolC<true>{});

  l = sum_pair32(l);
  // acc holds 256 * sum_t (r_t / r_last) sum_j p_j code_j 2^(e_t - e_max)
  const float fac = __builtin_amdgcn_ldexpf(r_cur, e_max) / l;
  // whole output rows through LDS (free after the last tile's barrier)
  store_tile_rows<false, D>(smem + wave * 32 * D * 2, acc, fac, lane, N - qw,
                            [&](int r) { return o + ((size_t)bh * N + qw + r) * D; });
  if (my_q < N && g == 0)
    lse[(size_t)bh * N + my_q] = (m + __builtin_amdgcn_logf(l) - kLog2PScale) * kLn2;
}

template <int NW2>
static hipError_t launch_fp8_dl(const FwdArgs& a) {
  const int nqt = (a.N + NW2 * 32 - 1) / (NW2 * 32);
  const long long blocks = (long long)nqt * a.B * a.H;
  const int BH = a.B * a.H;
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NW2 * 64), 0, (hipStream_t)a.stream,
                       (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, a.q_scale,
                       a.k_scale, a.v_scale, (bf16*)a.o, a.lse, BH, a.N, a.scale_log2);
  };
  if (a.causal)
    args(fa_fwd_fp8_dl_kernel<true, NW2>);
  else
    args(fa_fwd_fp8_dl_kernel<false, NW2>);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const FwdArgs& a) {
  if (a.d != D || a.out_f32) return hipErrorNotSupported;
  // direct loads, 128-key tiles, 4 waves: 1473 vs 1409 TFLOP/s for the
  // register-staged 64-key kernel at B=4 H=16 N=8192 causal (same process);
  // 8 waves: 1443
  return launch_fp8_dl<4>(a);
}

}  // namespace fa
