// FlashAttention forward pass, bf16 inputs, on gfx950 matrix cores.
//
// Method (the "Flash Attention" Markdown note, sections "Tiling（分块）技术"
// and "递归计算softmax"; loop order from the FlashAttention-2 overview):
// queries are tiled in the outer loop (a workgroup per two query tiles of
// one (batch, head)), keys/values in the inner loop.  For every key tile the
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
//    128-key K/V tile, double-buffered in LDS.  Tiles move from HBM to LDS
//    with direct buffer loads (no register staging, no LDS store
//    instructions), issued for tile j+1 while tile j is computed; rows past
//    N read as 0 through the buffer resource's range.  K and V are stored
//    row-major with the 16-byte chunks of each row XOR-swizzled (K by the
//    row index mod 16, V by 4 (2 at d = 64) times the row index mod 4) so that the MFMA
//    operand reads hit distinct LDS banks.  V^T operands are read with the
//    transposing ds_read_b64_tr_b16: lane j of each 16-lane group points at
//    one key row and four columns, and lane i receives one column over four
//    consecutive keys -- the order in which the score accumulator hands P^T
//    to the next MFMA.  Operand reads run four MFMAs ahead of their use.
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA.  The
//    reference max is only moved (and O, l rescaled) when a tile's weights
//    against it sum to 2^8 or more on some lane, which includes every tile
//    where a lane's max grows by more than 2^8; otherwise the stale
//    reference is kept, which leaves the result exact and skips most
//    rescales.  A tile's own max is only taken in those tiles, after its
//    weights were formed against the stale reference.  l sums the fp32
//    probabilities (before their bf16 rounding for the MFMA), so the stored
//    log-sum-exp carries no bf16 error even for rows with few keys.
//  * The epilogue stages each wave's 32 output rows in LDS and stores them
//    as whole rows (16 lanes per 256-byte row), not 8 bytes per row and
//    lane.
//  * Causal: key tiles entirely above the diagonal are never loaded; within
//    a workgroup, a wave whose 32 queries all precede a tile skips its math;
//    masking is applied only on tiles that straddle the diagonal or N.
//  * IEEE fp16 inputs (F16) take the same path with the fp16 MFMA: the
//    layouts, swizzles and transposing reads only see 16-bit elements.  P is
//    then rounded to fp16 (below 2^8 under the lazy rescale, so in range;
//    terms below 2^-24 of the reference are lost from P*V but not from l)
//    and O is stored as fp16 unless fp32 output is asked for.
//  * Packed batches of unequal lengths use the same kernel with runtime
//    strides: each workgroup finds its sequence's query and key rows from
//    the cumulative lengths, and causal masking is aligned at the sequence
//    end (query i sees key j iff j <= i + Lk - Lq).  A query that sees no
//    key gets O = 0 and LSE = -inf.
//  * A workgroup computes two query tiles of one (sequence, head), one
//    after the other: row r of the grid takes tiles nqt-1-r and r.  Under
//    causal masking their key spans add up to the same length in every
//    row, so the rows are balanced; the heavier tile runs first.  While the
//    first tile's last key tile is computed, the second tile's first key
//    tile is already loading into the other LDS stage, and its Q rows load
//    during the first tile's epilogue, so only the first tile of each
//    workgroup waits for its inputs.  Consecutive workgroups take different
//    heads, so with B*H a multiple of 8 every query tile of a head lands on
//    the same XCD (dispatch is round-robin over the 8 XCDs) and shares its
//    K/V in that XCD's L2.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

template <int D, int BC, int NW>
struct FwdCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BR = NW * 32;       // queries per workgroup
  static constexpr int KST = D;            // K row stride in LDS (bf16), unpadded
  static constexpr int VST = D;            // V row stride in LDS (bf16), unpadded
  static constexpr int KTILE = BC * KST;
  static constexpr int VTILE = BC * VST;
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shapes");
};

// Where one (sequence, head) lives.  Dense: [B, H, N, d] with N keys per
// query row set.  Packed: [total, H, d] rows with cumulative lengths.
struct FwdLayout {
  const int* cu_q;     // null for dense
  const int* cu_k;
  int H, N, Nk, total_q, total_k;   // N, Nk: longest query / key sequence
};

template <int D, int BC, int NW, bool CAUSAL, bool OUT_F32, bool F16>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
__attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                        const bf16* __restrict__ v, void* __restrict__ o,
                        float* __restrict__ lse, int BH, FwdLayout lay,
                        float c /* scale*log2(e) */) {
  using C = FwdCfg<D, BC, NW>;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (C::KTILE + C::VTILE)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index as a uniform value, so that the LDS targets of the
  // direct loads are computed in scalar registers (no per-load
  // v_readfirstlane into M0)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  const int bh = blockIdx.x % BH;
  int qt = blockIdx.x / BH;
  // this (sequence, head): first rows, lengths, row stride and LSE offset
  int Lq = lay.N, Lk = lay.N, rs = D;
  size_t qbase, kbase, lbase;
  if (lay.cu_q) {
    const int b = bh / lay.H, h = bh % lay.H;
    const int sq = min(max(lay.cu_q[b], 0), lay.total_q);
    const int sk = min(max(lay.cu_k[b], 0), lay.total_k);
    Lq = min(max(min(lay.cu_q[b + 1], lay.total_q) - sq, 0), lay.N);
    Lk = min(max(min(lay.cu_k[b + 1], lay.total_k) - sk, 0), lay.Nk);
    rs = lay.H * D;
    qbase = (size_t)sq * rs + (size_t)h * D;
    kbase = (size_t)sk * rs + (size_t)h * D;
    lbase = (size_t)h * lay.total_q + sq;
  } else {
    qbase = kbase = (size_t)bh * (size_t)lay.N * D;
    lbase = (size_t)bh * lay.N;
  }
  const int nqt = (Lq + C::BR - 1) / C::BR;
  // Row r of the grid takes query tiles nqt-1-r and r of this (sequence,
  // head), in that order: under causal masking their KV spans add up to the
  // same length in every row, and the second tile's first K/V tile and Q
  // rows are fetched while the first one finishes.
  const int row = qt;
  if (row >= (nqt + 1) / 2) return;         // past this sequence's queries (whole workgroup)
  const int nitems = nqt - 1 - row > row ? 2 : 1;
  const int off = CAUSAL ? Lk - Lq : 0;     // causal: query i sees keys j <= i + off
  const bf16* Qh = q + qbase;
  const bf16* Kh = k + kbase;
  const bf16* Vh = v + kbase;
  const uint32_t RG = (uint32_t)rs * 2u;    // bytes from one row to the next in HBM

  qt = nqt - 1 - row;

  const rsrc_t Qr = make_rsrc(Qh, (uint32_t)Lq * RG);
  [[maybe_unused]] const rsrc_t Kr = make_rsrc(Kh, (uint32_t)Lk * RG);
  [[maybe_unused]] const rsrc_t Vr = make_rsrc(Vh, (uint32_t)Lk * RG);
  bf16x8 qb[D / 16];
  auto load_q = [&](int t) {
    const int mq = t * C::BR + wave * 32 + l32;
#pragma unroll
    for (int u = 0; u < D / 16; ++u)
      qb[u] = __builtin_bit_cast(bf16x8, buf_load16(Qr, (uint32_t)mq * RG + (16u * u + 8u * g) * 2u));
  };
  auto tiles_of = [&](int t) {
    const int kv_end = CAUSAL ? max(0, min(Lk, t * C::BR + C::BR + off)) : Lk;
    return (kv_end + BC - 1) / BC;
  };
  load_q(qt);

  // Direct global -> LDS loads.  One wave instruction fills 1 KB of LDS
  // (lane i -> bytes 16i..16i+15); the 16-byte chunk c of row r sits at
  // chunk position c ^ (r % NCH) for K and c ^ VS(r % 4) for V, so the MFMA
  // reads below hit distinct banks.  Each lane's global offset carries the
  // inverse permutation.
  constexpr int RB = D * 2;                      // bytes per row
  constexpr int NCH = RB / 16;                   // chunks per row
  // V's swizzle step.  A transposing read serves 32 lanes at a time: four
  // rows (r % 4 = 0..3) times one aligned group of four 16-byte chunks.  At
  // d = 128 a row is 256 bytes, every bank once, so the four rows' groups
  // must land on four different groups of chunk positions: XOR by 4(r % 4).
  // (XOR by 2(r % 4) put rows r and r ^ 1 on the same banks: a two-way
  // conflict on every V^T read.)  At d = 64 two rows share the banks' width
  // and 2(r % 4) is conflict-free.
  constexpr int VS = D == 128 ? 4 : 2;
  constexpr int NI = BC * RB / 1024;             // 1 KB instructions per tile
  constexpr int IPW = NI / NW;                   // per wave, for K and for V each
  static_assert(NI % NW == 0 && NCH >= 8, "direct-load tiling");
  uint32_t gk[IPW], gv[IPW];
#pragma unroll
  for (int x = 0; x < IPW; ++x) {
    const int blk = wave * IPW + x;
    const int byte = blk * 1024 + lane * 16;
    const int r = byte / RB, p = (byte % RB) / 16;
    gk[x] = (uint32_t)r * RG + (uint32_t)(16 * (p ^ (r % NCH)));
    gv[x] = (uint32_t)r * RG + (uint32_t)(16 * (p ^ (VS * (r & 3))));
  }
  // key tile j into LDS stage st
  auto load_tile = [&](int j, int st) {
    [[maybe_unused]] const uint32_t tile = (uint32_t)j * BC * RG;
    uint8_t* Kd = reinterpret_cast<uint8_t*>(smem + (st & 1) * (C::KTILE + C::VTILE));
    [[maybe_unused]] uint8_t* Vd = Kd + C::KTILE * 2;
#if defined(__HIP_DEVICE_COMPILE__)  // the LDS-DMA builtin exists in the device pass only
#pragma unroll
    for (int x = 0; x < IPW; ++x) {
      const int blk = wave * IPW + x;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Kr, (__attribute__((address_space(3))) void*)(Kd + blk * 1024), 16, tile + gk[x], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Vr, (__attribute__((address_space(3))) void*)(Vd + blk * 1024), 16, tile + gv[x], 0, 0, 0);
    }
#endif
  };
  auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0)

  // per-lane LDS read offsets (bytes within a tile).  K: row l32 (+32b),
  // logical chunk 2u + g.  V (transposing reads): lane j of a 16-lane group
  // reads row 4g + j/4 (+16t, +8), columns 32cb + 16dh + 4(j%4), i.e.
  // logical chunk 4cb + 2dh + (j%4)/2 and byte 8(j%2) inside it.
  uint32_t k_rd[D / 16], v_rd[D / 32];
#pragma unroll
  for (int u = 0; u < D / 16; ++u)
    k_rd[u] = (uint32_t)(l32 * RB + 16 * ((2 * u + g) ^ (l32 % NCH)));
  {
    const int j16 = lane & 15, dh = (lane >> 4) & 1, q4 = j16 >> 2;
    const int r = 4 * g + q4;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      const int c = 4 * cb + 2 * dh + ((j16 & 3) >> 1);
      v_rd[cb] = (uint32_t)(r * RB + 16 * (c ^ (VS * (r & 3))) + 8 * (j16 & 1));
    }
  }
  int gt = 0;                // tiles computed so far (LDS stage = gt & 1)
  int ntiles = tiles_of(qt);
  bool loaded = false;       // the current query tile's first key tile is in stage gt & 1

  for (int item = 0; item < nitems; ++item) {
    if (item == 1) qt = row;
    if (!loaded) {
      if (ntiles > 0) load_tile(0, gt);
      wait_loads();            // also the Q rows
      __syncthreads();
    }
    const int q0 = qt * C::BR;
    const int qw = q0 + wave * 32;   // first query of this wave
    const int my_q = qw + l32;       // the query this lane's columns belong to
    const int ntiles_next = item + 1 < nitems ? tiles_of(row) : 0;
    f32x16 acc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};
    float m = kNegInf;   // reference max, base-2 units of the scaled scores
    float l = 0.f;       // this lane's share of the row sum (keys of its half)

    for (int j = 0; j < ntiles; ++j, ++gt) {
      const int buf = gt & 1;
      // the next tile of this query tile, or the first of the next one
      const bool more = j + 1 < ntiles || ntiles_next > 0;
      if (more) load_tile(j + 1 < ntiles ? j + 1 : 0, gt + 1);
      loaded = more;

      const int kb = j * BC;
      // a wave past its sequence's queries, or wholly before this tile's keys, skips the math
      const bool active = qw < Lq && (!CAUSAL || kb <= qw + 31 + off);
      if (active) {
        const bf16* Ks = smem + buf * (C::KTILE + C::VTILE);
        const bf16* Vs = Ks + C::KTILE;

        // ---- S^T = K * Q^T : keys on rows, this lane's query on the column ----
        f32x16 s[BC / 32];
#pragma unroll
        for (int b = 0; b < BC / 32; ++b) s[b] = f32x16{};
        {
          // K fragments are read PD MFMAs ahead of their use; the scheduling
          // fence after every step keeps the compiler from sinking each read
          // next to its MFMA (which leaves only two LDS reads in flight)
          constexpr int PDK = 4;
          constexpr int NB = BC / 32, NQ = (D / 16) * NB;
          bf16x8 kf[NQ];
#pragma unroll
          for (int i = 0; i < NQ + PDK; ++i) {
            if (i < NQ) {
              const int u = i / NB, b = i % NB;
              kf[i] = *reinterpret_cast<const bf16x8*>(
                  reinterpret_cast<const uint8_t*>(Ks) + (32 * b) * RB + k_rd[u]);
            }
            if (i >= PDK) {
              const int x = i - PDK, u = x / NB, b = x % NB;
              s[b] = mma16<F16>(kf[x], qb[u], s[b]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }

        // ---- mask keys past the diagonal or past N (edge tiles only) ----
        const bool edge = (CAUSAL && kb + BC - 1 > qw + off) || kb + BC > Lk;
        if (edge) {
#pragma unroll
          for (int b = 0; b < BC / 32; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kb + 32 * b + 8 * (i >> 2) + 4 * g + (i & 3);
              const bool dead = key >= Lk || (CAUSAL && key > my_q + off);
              s[b][i] = dead ? kNegInf : s[b][i];
            }
        }

        // ---- online softmax (base 2) ----
        // The tile is exponentiated against the reference max m without first
        // taking its own max.  Its weights may then exceed 1 (exact in fp32
        // and bf16); a tile whose weights sum to 2^8 or more on some lane
        // (any weight above 2^8 among them, i.e. a max that grew by more than
        // 8 in base 2), or a lane with no reference yet, takes the tile max,
        // moves the reference there (O and l rescaled) and forms its weights
        // again.  So the reference moves at least whenever the max-based lazy
        // rule would move it, and the max over every score of a tile is taken
        // only in those rare tiles.
        const float l_in = l;
        bf16x8 pb[BC / 16];
        auto form_p = [&](float mref) __attribute__((always_inline)) {
#pragma unroll
          for (int t = 0; t < BC / 16; ++t) {
            uint32_t w[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              const float p0 = __builtin_amdgcn_exp2f(fmaf(s[t >> 1][8 * (t & 1) + 2 * h], c, -mref));
              const float p1 = __builtin_amdgcn_exp2f(fmaf(s[t >> 1][8 * (t & 1) + 2 * h + 1], c, -mref));
              w[h] = pack16<F16>(p0, p1);
              l += p0 + p1;
            }
            pb[t] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
          }
        };
        form_p(m == kNegInf ? 0.f : m);
        if (__builtin_amdgcn_ballot_w64(!(l - l_in < 256.f) || m == kNegInf)) {
          float mx = kNegInf;
#pragma unroll
          for (int b = 0; b < BC / 32; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[b][i]);
          mx = max_pair32(mx) * c;
          const float m_cand = fmaxf(m, mx);
          const float alpha = (m_cand == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m - m_cand);
          m = m_cand;
#pragma unroll
          for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[cb][i] *= alpha;
          l = l_in * alpha;
          form_p(m == kNegInf ? 0.f : m);
        }

        // ---- O^T += V^T * P^T ----
        {
          // V^T fragments, read PDV MFMAs ahead as for K
          typedef short s16x4 __attribute__((ext_vector_type(4)));
          constexpr int PDV = 4;
          constexpr int NC = D / 32, NV = (BC / 16) * NC;
          bf16x8 vf[NV];
#pragma unroll
          for (int i = 0; i < NV + PDV; ++i) {
            if (i < NV) {
              const int t = i / NC, cb = i % NC;
              const uint8_t* vp = reinterpret_cast<const uint8_t*>(Vs) + (16 * t) * RB + v_rd[cb];
              const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) s16x4*)(vp));
              const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) s16x4*)(vp + 8 * RB));
              vf[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
            if (i >= PDV) {
              const int x = i - PDV, t = x / NC, cb = x % NC;
              acc[cb] = mma16<F16>(vf[x], pb[t], acc[cb]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }

      if (more) wait_loads();
      __syncthreads();
    }

    // the epilogue's per-lane addresses are computed here, not kept live
    // across the loops (the compiler would hoist them out of the item loop)
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    // the next query tile's Q rows, while this one is stored
    if (item + 1 < nitems) load_q(row);

    // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2 (0 and -inf for a
    // query that saw no key) ----
    l = sum_pair32(l);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if constexpr (OUT_F32) {
      if (my_q < Lq) {
        const size_t orow = qbase + (size_t)my_q * rs;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int d0 = 32 * cb + 8 * ii + 4 * g;
            *reinterpret_cast<f32x4*>(static_cast<float*>(o) + orow + d0) =
                f32x4{acc[cb][4 * ii] * inv, acc[cb][4 * ii + 1] * inv, acc[cb][4 * ii + 2] * inv,
                      acc[cb][4 * ii + 3] * inv};
          }
      }
    } else {
      // 16-bit output: whole rows through LDS (free after the last tile's
      // barrier), 8 KB per wave
      bf16* ob = static_cast<bf16*>(o);
      // staged in the LDS stage of the last tile, not the one holding the
      // next query tile's first key tile
      store_tile_rows<F16, D>(reinterpret_cast<uint8_t*>(smem + ((gt + 1) & 1) * (C::KTILE + C::VTILE)) + wave * 32 * RB,
                              acc, inv, lane_e, Lq - qw,
                              [&](int r) { return ob + qbase + (size_t)(qw + r) * rs; });
    }
    if (my_q < Lq && g == 0) lse[lbase + my_q] = l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : kNegInf;
    ntiles = ntiles_next;
    if (item + 1 < nitems) __syncthreads();   // staging read back before the next tile loads land
  }
}

template <int D, int BC, int NW, bool CAUSAL, bool OUT_F32, bool F16>
static hipError_t launch(const FwdArgs& a) {
  using C = FwdCfg<D, BC, NW>;
  const int nqt = (a.N + C::BR - 1) / C::BR;   // of the longest sequence
  const long long blocks = (long long)((nqt + 1) / 2) * a.B * a.H;   // two query tiles per workgroup
  const FwdLayout lay{a.cu_q, a.cu_k, a.H, a.N, a.Nk, a.total_q, a.total_k};
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, BC, NW, CAUSAL, OUT_F32, F16>), dim3((unsigned)blocks),
                     dim3(C::NT), 0, (hipStream_t)a.stream, (const bf16*)a.q, (const bf16*)a.k,
                     (const bf16*)a.v, a.o, a.lse, a.B * a.H, lay, a.scale_log2);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool OUT_F32>
static hipError_t launch_d(const FwdArgs& a) {
  if (a.in_f16) return launch<D, 128, 8, CAUSAL, OUT_F32, true>(a);
  return launch<D, 128, 8, CAUSAL, OUT_F32, false>(a);
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
