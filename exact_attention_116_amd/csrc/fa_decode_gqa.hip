// Split-KV single-query decode with grouped key/value heads (GQA; MQA when
// there is a single key/value head).
//
// Method: as the plain split-KV decode (the FlashAttention-2 overview's
// two-part K/V split example generalised to num_splits ranges, merged with
// the FlashAttention-3 snippets' splitK combine), except that G = Hq / Hkv
// query heads read the same cached K/V head (the MQA note among the related
// posts of the CSDN "flash attention CUDA programming, pipeline-parallel
// acceleration V6" page: keys and values keep one shared head, queries keep
// all of theirs).  One workgroup takes one (batch, K/V head, split) and up to
// 16 (groups of at most 16) or 32 (larger groups) of the query heads that
// share it, so every cached byte it streams serves all of them.  With a
// length per sequence, sequence b uses the first seqlens[b] keys of its
// padded cache, split into num_splits ranges of its own.
//
// gfx950 mapping: the G queries of a group make both products small dense
// contractions, so they run on v_mfma_f32_16x16x32_bf16 with the query heads
// on the 16-wide N side:
//   S^T (16 keys x 16 heads) = K (16 keys x 32 d) * Q^T, 4 k-steps at d=128;
//   O^T (16 d    x 16 heads) += V^T (16 d x 32 keys) * P^T.
// Each lane therefore owns one query head (column l%16) and the same head's
// online-softmax state, so P^T goes from the score accumulators straight into
// the B operand of the second product.  The K rows of a 32-key step are read
// in an order chosen so that the score layout (lane group g = l/16 holds keys
// 8g+4b+i of score block b) equals the B-operand order of P^T (lane group g
// supplies keys 8g..8g+7).  V is read row-wise, fully coalesced (16 lanes
// cover one 256-byte row), and transposed in registers with v_perm_b32 into
// the V^T A operand; output row m of block i is feature d = (D/16)*m + i, so
// at the end a lane holds 4*D/16 consecutive features of its head.  The
// streaming is the whole cost; the matrix cores run far below their rate.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

template <int D, int NW, int U, int QB>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
void fa_decode_gqa_split_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kc,
                                const bf16* __restrict__ vc, float* __restrict__ part_o,
                                float* __restrict__ part_lse, const int* __restrict__ seqlens,
                                int Hq, int Hkv, int G, int QC, int Lkv, int S, int chunk,
                                float c) {
  static_assert(D == 64 || D == 128, "head dimension 64 or 128");
  constexpr int KT = D / 32;    // k-steps of the score product
  constexpr int NB = D / 16;    // 16-feature blocks of the output; also features per lane of a V row
  constexpr int NH = 16 * QB;   // query heads per workgroup (QB blocks of 16)
  constexpr int STEP = 32;      // keys per MFMA step
  constexpr int WSTEP = NW * U * STEP;
  constexpr float kLazy = 8.f;  // move the reference max only when it grows by > 2^8
  __shared__ float sm_m[NW][NH], sm_l[NW][NH];
  __shared__ float sm_o[NW][NH][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int s = blockIdx.x % S;
  const int rest = blockIdx.x / S;
  const int qc = rest % QC;
  const int bkv = rest / QC;  // b * Hkv + kv head
  const int b = bkv / Hkv, hk = bkv % Hkv;
  const int h0 = hk * G + qc * NH;
  const int gc = (G - qc * NH) < NH ? (G - qc * NH) : NH;  // query heads of this workgroup

  // keys of this sequence: all Lkv, or its own length within the padded
  // cache, cut into S splits of ceil(length / S)
  int Lb = Lkv;
  if (seqlens) {
    Lb = min(max(seqlens[b], 0), Lkv);
    chunk = (Lb + S - 1) / S;
  }
  const long long lo_ll = (long long)s * chunk;
  const int lo = (int)(lo_ll < Lb ? lo_ll : Lb);
  const int hi = (int)((long long)lo + chunk < Lb ? (long long)lo + chunk : Lb);
  const int nkeys = hi - lo;

  // Q^T as the B operand of the score product: column n of block qq is query
  // head h0 + 16*qq + n, contraction slots d = 32t + 8g + j.  Heads past the
  // group read as zero.
  bf16x8 qb[QB][KT];
#pragma unroll
  for (int qq = 0; qq < QB; ++qq) {
    const int hn = 16 * qq + n;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const bf16* qp = q + ((size_t)b * Hq + (size_t)(h0 + (hn < gc ? hn : 0))) * D + 8 * g;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const u32x4 w = (hn < gc) ? *reinterpret_cast<const u32x4*>(qp + 32 * t) : z;
      qb[qq][t] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // K/V rows of this split through buffer resources spanning exactly
  // [lo, hi): rows past hi read as 0 (their scores are masked to -inf).
  const size_t head = ((size_t)bkv * (size_t)Lkv + (size_t)lo) * D;
  const uint32_t span = (uint32_t)nkeys * D * 2u;
  const rsrc_t Kr = make_rsrc(kc + head, span);
  const rsrc_t Vr = make_rsrc(vc + head, span);

  // key of A-operand row n in score block bb of a 32-key step
  const int krow0 = 8 * (n >> 2) + (n & 3);
  float mref[QB], lsum[QB];
  f32x4 acc[QB][NB];
#pragma unroll
  for (int qq = 0; qq < QB; ++qq) {
    mref[qq] = kNegInf;
    lsum[qq] = 0.f;
#pragma unroll
    for (int i = 0; i < NB; ++i) acc[qq][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int kb0 = 0; kb0 < nkeys; kb0 += WSTEP) {
    u32x4 kr[U][2][KT];
    uint32_t vr[U][8][NB / 2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kb0 + (u * NW + wave) * STEP;
      // A K load instruction covers 64 bytes of each of 16 rows, half of a
      // 128-byte cache line, and the next one the other half: without the
      // non-temporal hint the line stays in L2 between the two, so the
      // cache is fetched once (with it, 3.6% of K was fetched twice and the
      // kernel streamed 5% slower).  V rows are read whole, non-temporally.
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int t = 0; t < KT; ++t)
          kr[u][bb][t] = buf_load16(Kr, ((uint32_t)(kb + krow0 + 4 * bb) * D + 32 * t + 8 * g) * 2u);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint32_t off = ((uint32_t)(kb + 8 * g + r) * D + NB * n) * 2u;
        if constexpr (NB == 8) {
          const u32x4 w = buf_load16_nt(Vr, off);
#pragma unroll
          for (int e = 0; e < 4; ++e) vr[u][r][e] = w[e];
        } else {
          const u32x2 w = buf_load8_nt(Vr, off);
          vr[u][r][0] = w[0];
          vr[u][r][1] = w[1];
        }
      }
    }

    // P^T of every head block and sub-step: slot j = 4*bb + i holds key 8g + j
    bf16x8 pb[QB][U];
#pragma unroll
    for (int qq = 0; qq < QB; ++qq) {
      // scores (log2 domain), masked past the end of the split
      float sc[U][2][4];
      float mx = kNegInf;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kb = kb0 + (u * NW + wave) * STEP;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < KT; ++t)
            a = mfma16x16x32(__builtin_bit_cast(bf16x8, kr[u][bb][t]), qb[qq][t], a);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sc[u][bb][i] = (kb + 8 * g + 4 * bb + i < nkeys) ? a[i] * c : kNegInf;
            mx = fmaxf(mx, sc[u][bb][i]);
          }
        }
      }
      // the four lane groups holding one head agree on its maximum
      mx = max_pair16(mx);
      mx = max_pair32(mx);
      if (mx > mref[qq] + kLazy) {
        const float alpha = __builtin_amdgcn_exp2f(mref[qq] - mx);  // 0 while mref = -inf
        mref[qq] = mx;
        lsum[qq] *= alpha;
#pragma unroll
        for (int i = 0; i < NB; ++i) acc[qq][i] *= alpha;
      }
      const float mb = (mref[qq] == kNegInf) ? 0.f : mref[qq];  // every score is -inf while mref is
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float p[2][4];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[bb][i] = __builtin_amdgcn_exp2f(sc[u][bb][i] - mb);
            lsum[qq] += p[bb][i];
          }
        const u32x4 pw = {pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                          pack_bf16(p[1][0], p[1][1]), pack_bf16(p[1][2], p[1][3])};
        pb[qq][u] = __builtin_bit_cast(bf16x8, pw);
      }
    }

    // V^T block i (row n is feature NB*n + i, slot j is key 8g + j), built
    // once and used by every head block
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        u32x4 vt;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp)
          vt[pp] = __builtin_amdgcn_perm(vr[u][2 * pp + 1][i >> 1], vr[u][2 * pp][i >> 1], sel);
#pragma unroll
        for (int qq = 0; qq < QB; ++qq)
          acc[qq][i] = mfma16x16x32(__builtin_bit_cast(bf16x8, vt), pb[qq][u], acc[qq][i]);
      }
  }

  // the row sum of a head is spread over its four lane groups
#pragma unroll
  for (int qq = 0; qq < QB; ++qq) {
    const float ls = sum_pair32(sum_pair16(lsum[qq]));
    if (g == 0) {
      sm_m[wave][16 * qq + n] = mref[qq];
      sm_l[wave][16 * qq + n] = ls;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm_o[wave][16 * qq + n][NB * (4 * g + r) + i] = acc[qq][i][r];
  }
  __syncthreads();

  // merge the waves' states and write each head's partial
  for (int idx = tid; idx < gc * D; idx += NW * 64) {
    const int hn = idx / D, dd = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][hn]);
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float wt = __builtin_amdgcn_exp2f(sm_m[w][hn] - M);  // -inf -> 0
        L = fmaf(wt, sm_l[w][hn], L);
        O = fmaf(wt, sm_o[w][hn][dd], O);
      }
    }
    const size_t ps = ((size_t)b * Hq + (size_t)(h0 + hn)) * S + s;
    part_o[ps * D + dd] = (M == kNegInf) ? 0.f : O / L;
    if (dd == 0) part_lse[ps] = (M == kNegInf) ? kNegInf : (M + __builtin_amdgcn_logf(L)) * kLn2;
  }
}

template <int D, int NW, int U, int QB>
static hipError_t launch_gqa_cfg(const DecodeArgs& a) {
  const int G = a.H / a.Hkv;
  const int QC = (G + 16 * QB - 1) / (16 * QB);
  const int chunk = (int)(((long long)a.Lkv + a.num_splits - 1) / a.num_splits);
  const long long grid = (long long)a.B * a.Hkv * QC * a.num_splits;
  hipLaunchKernelGGL((fa_decode_gqa_split_kernel<D, NW, U, QB>), dim3((unsigned)grid), dim3(NW * 64),
                     0, (hipStream_t)a.stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
                     a.part_o, a.part_lse, a.seqlens_k, a.H, a.Hkv, G, QC, a.Lkv, a.num_splits,
                     chunk, a.scale_log2);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_gqa_d(const DecodeArgs& a) {
  // groups of more than 16 heads take 32 per workgroup, so each K/V byte is
  // streamed once for up to 32 query heads
  const int G = a.H / a.Hkv;
  // (one 32-key step per wave and iteration: the lower register count buys
  // more resident waves, which streams faster than deeper unrolling)
  hipError_t e = (G > 16) ? launch_gqa_cfg<D, 4, 1, 2>(a) : launch_gqa_cfg<D, 4, 1, 1>(a);
  if (e != hipSuccess) return e;
  return launch_decode_combine(a);
}

hipError_t launch_decode_gqa(const DecodeArgs& a) {
  return a.d == 128 ? launch_gqa_d<128>(a) : launch_gqa_d<64>(a);
}

}  // namespace fa
