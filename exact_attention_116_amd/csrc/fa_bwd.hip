// FlashAttention backward pass (dQ, dK, dV), bf16, on gfx950 matrix cores.
//
// Method: the gradients of O = softmax(scale * Q K^T) V for an upstream dO,
// with P recomputed from Q, K and the log-sum-exp the forward pass saved
// instead of a stored score matrix (the recomputation named in the
// FlashAttention summaries; the pages split the backward pass over thread
// blocks in their own way in the FlashAttention-2 overview, section 3.4, and
// keep the softmax statistics in fp32, "使用注意事项" of the Flash Attention
// note):
//     P  = exp(scale * Q K^T - LSE)          dV = P^T dO
//     dP = dO V^T                            dS = P * (dP - D),  D = rowsum(dO * O)
//     dQ = scale * dS K                      dK = scale * dS^T Q
// (D equals rowsum(P * dP), the softmax Jacobian's correction term, because
// O = P V.)
//
// IEEE fp16 tensors (F16) take the same kernels with the fp16 MFMA and fp16
// roundings of P and dS; the statistics stay fp32.
//
// Packed batches of unequal lengths (PACKED instances) use the same kernels
// with runtime row strides: [total, H, d] rows, LSE and the row arrays of
// the workspace as [H, total_q],
// each workgroup's sequence found from the cumulative lengths, and causal
// masking aligned at the sequence end (query i sees key j iff
// j <= i + Lk - Lq).  A query that sees no key gets dQ = 0; keys of a
// sequence without queries get dK = dV = 0.
//
// Three kernels, none of which needs atomics (so the result is
// deterministic):
//  1. fa_bwd_pre_kernel: per query row, -D (fp32, from bf16 O and dO) and
//     -LSE/scale, the starting values of the dK/dV kernel's accumulators.
//  2. fa_bwd_dkdv_kernel: key/value tiles outer, query tiles inner.  A pair
//     of waves owns 32 keys; K^T (one wave) and V^T (the other) stay in
//     VGPRs as MFMA B operands.  Per 32-query block one wave forms
//     S = Q K^T, P and dV^T += dO^T P, the other dP = dO V^T, then, with P
//     handed over through LDS, dS and dK^T += Q^T dS (one key per lane
//     column; P and dS go straight in as B operands).  Each block's second
//     product is deferred by one block, so that it overlaps the next
//     block's exponentials and dS work.
//  3. fa_bwd_dq_kernel: query tiles outer, key/value tiles inner, the
//     forward kernel's layout: Q^T and dO^T stay in VGPRs, one query per lane
//     column, S^T = K Q^T and dP^T = V dO^T, then dQ^T += K^T dS^T.
// Recomputing S and dP in the dQ kernel costs 40% more matrix work than
// accumulating dQ across key tiles with fp32 atomics, which would move
// several GB of atomic traffic per launch at these sizes.
//
// LDS: tiles arrive by direct global->LDS buffer loads, double-buffered.
// Q and dO (kernel 2) and K (kernel 3) are read both row-wise (16-byte
// fragments of one row per lane) and transposed (ds_read_b64_tr_b16), so
// their 16-byte chunks are XOR-swizzled with a pattern that keeps both
// reads free of bank conflicts: at 256 bytes per row, chunk c of row r sits
// at c ^ (4*(r%4) + (r/4)%4).
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// XOR swizzle of the 16-byte chunks of LDS row r (RB bytes per row).
template <int RB>
__device__ __forceinline__ int bwd_swz(int r) {
  static_assert(RB == 256 || RB == 128, "rows of 64 or 128 bf16");
  if constexpr (RB == 256) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Direct global->LDS copy of ROWS rows of RB bytes, swizzled; NW waves share
// the 1 KB instructions.  Rows are RG bytes apart in memory (RB for a dense
// [.., N, d] head, H*d*2 for packed [total, H, d] rows) and RB apart in LDS.
// base_off is the byte offset of the tile's first row in the buffer resource.
template <int RB, int ROWS, int NW>
struct TileLoader {
  static constexpr int NI = ROWS * RB / 1024;
  static constexpr int IPW = NI / NW;
  static_assert(NI % NW == 0, "tile must split evenly over the waves");
  uint32_t goff[IPW];
  __device__ __forceinline__ void init(int wave, int lane, uint32_t RG) {
#pragma unroll
    for (int x = 0; x < IPW; ++x) {
      const int byte = (wave * IPW + x) * 1024 + lane * 16;
      const int r = byte / RB, p = (byte % RB) / 16;
      goff[x] = (uint32_t)r * RG + (uint32_t)(16 * (p ^ bwd_swz<RB>(r)));
    }
  }
  __device__ __forceinline__ void load(rsrc_t R, uint32_t base_off, uint8_t* lds, int wave) const {
#pragma unroll
    for (int x = 0; x < IPW; ++x) lds_dma16(R, lds + (wave * IPW + x) * 1024, base_off + goff[x]);
  }
};

__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Per-lane LDS byte offsets for the two read patterns of a swizzled tile.
//  row:  A operand of a 32x32x16 MFMA from row-major data: lane l reads row
//        l%32 (+32 per block), bf16 columns 16u + 8(l/32) .. +7.
//  tr:   A operand built from the transpose: two ds_read_b64_tr_b16 (rows
//        +0 and +8 of a 16-row step) give lane l column 32cb + l%32 over the
//        eight rows in the order of a 32x32 accumulator's row index.
template <int D>
struct TileReads {
  static constexpr int RB = D * 2;
  uint32_t row[D / 16];
  uint32_t tr_lo[D / 32], tr_hi[D / 32];
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
    for (int u = 0; u < D / 16; ++u)
      row[u] = (uint32_t)(l32 * RB + 16 * ((2 * u + g) ^ bwd_swz<RB>(l32)));
    const int j16 = lane & 15, dh = (lane >> 4) & 1, q4 = j16 >> 2;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      const int c = 4 * cb + 2 * dh + ((j16 & 3) >> 1);
      const int rl = 4 * g + q4, rh = rl + 8;
      tr_lo[cb] = (uint32_t)(rl * RB + 16 * (c ^ bwd_swz<RB>(rl)) + 8 * (j16 & 1));
      tr_hi[cb] = (uint32_t)(rh * RB + 16 * (c ^ bwd_swz<RB>(rh)) + 8 * (j16 & 1));
    }
  }
  // row fragment u of the 32-row block starting at row r0 (a multiple of 32)
  __device__ __forceinline__ bf16x8 rowfrag(const uint8_t* t, int r0, int u) const {
    return *reinterpret_cast<const bf16x8*>(t + r0 * RB + row[u]);
  }
  // transposed fragment: rows r0 .. r0+15 (r0 a multiple of 16), columns 32cb..
  __device__ __forceinline__ bf16x8 trfrag(const uint8_t* t, int r0, int cb) const {
    const uint8_t* b = t + r0 * RB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(b + tr_lo[cb]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(b + tr_hi[cb]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// Where one (sequence, head) lives.  Dense: [B, H, N, d] tensors, LSE and D
// [B*H, N].  Packed (cu_q non-null): [total, H, d] token-major rows, LSE and
// D [H, total_q], sequence b at rows cu_q[b].. (queries) and cu_k[b]..
// (keys); N and Nk bound the query and key lengths.
struct BwdLayout {
  const int* cu_q;
  const int* cu_k;
  int H, N, Nk, total_q, total_k;
};

struct BwdSeq {
  size_t qbase, kbase, lbase;   // elements: first Q (and dO, O, dQ) row, first K row; LSE/D offset
  int Lq, Lk, rs;               // lengths, row stride in elements
};

template <int D, bool PACKED>
__device__ __forceinline__ BwdSeq bwd_seq(const BwdLayout& lay, int bh) {
  BwdSeq r;
  if constexpr (PACKED) {
    const int b = bh / lay.H, h = bh % lay.H;
    // the offsets as uniform values (scalar registers: the tile and block
    // decisions below stay scalar branches), clamped to the tensors, so that
    // malformed offsets give wrong values, never accesses outside them
    const int q0 = __builtin_amdgcn_readfirstlane(lay.cu_q[b]);
    const int q1 = __builtin_amdgcn_readfirstlane(lay.cu_q[b + 1]);
    const int k0 = __builtin_amdgcn_readfirstlane(lay.cu_k[b]);
    const int k1 = __builtin_amdgcn_readfirstlane(lay.cu_k[b + 1]);
    const int sq = min(max(q0, 0), lay.total_q);
    const int sk = min(max(k0, 0), lay.total_k);
    r.Lq = min(max(min(q1, lay.total_q) - sq, 0), lay.N);
    r.Lk = min(max(min(k1, lay.total_k) - sk, 0), lay.Nk);
    r.rs = lay.H * D;
    r.qbase = (size_t)sq * r.rs + (size_t)h * D;
    r.kbase = (size_t)sk * r.rs + (size_t)h * D;
    r.lbase = (size_t)h * lay.total_q + sq;
  } else {
    r.Lq = r.Lk = lay.N;
    r.rs = D;
    r.qbase = r.kbase = (size_t)bh * (size_t)lay.N * D;
    r.lbase = (size_t)bh * lay.N;
  }
  return r;
}

// ---------------------------------------------------------------------------
// 1. -D = -rowsum(dO * O), and -LSE/scale
// ---------------------------------------------------------------------------
// Rows are contiguous d-element rows of O and dO.  Dense: row r is (b*H+h)*N
// + n and its values go to index r.  Packed (H > 0): row r is token r/H, head
// r%H, at index (r%H) * total_q + r/H ([H, total_q], the LSE layout).  Both
// values are the starting values of the dK/dV kernel's accumulators, stored
// so that its loop takes them as loaded (16 VALU operations fewer per
// 32-query block and wave).
template <int D, bool F16>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void fa_bwd_pre_kernel(const bf16* __restrict__ o, const bf16* __restrict__ dout,
                       const float* __restrict__ lse, float* __restrict__ ndsum,
                       float* __restrict__ nlse, long long rows, int H, int total_q,
                       float neg_inv_scale) {
  constexpr int LPR = D / 8;  // lanes per row, 16 bytes each
  const long long row = (long long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + row * D + 8 * part);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dout + row * D + 8 * part);
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = dot2_16<F16>(a[w], b[w], acc);
  }
  acc = group_sum<LPR>(acc);
  if (row < rows && part == 0) {
    const long long at = H > 0 ? (long long)(row % H) * total_q + row / H : row;
    ndsum[at] = -acc;
    nlse[at] = lse[at] * neg_inv_scale;
  }
}

// ---------------------------------------------------------------------------
// 2. dK, dV: key tiles outer, each 32-key block's work split over a pair of waves
// ---------------------------------------------------------------------------
// Barrier over the workgroup's LDS reads and writes only: unlike
// __syncthreads (and unlike a workgroup fence on LDS, which also waits for
// the direct global->LDS loads) it does not wait for this wave's buffer
// loads, so a tile prefetch into the other LDS stage stays in flight across
// it.  The signal fences keep the compiler from moving memory accesses
// across the barrier; lgkmcnt(0) completes this wave's LDS accesses.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// A pair of waves owns 32 keys; the two halves of the block's work run on
// its two waves.  Role 0 holds K^T as MFMA B operands and forms S = Q K^T,
// P, and dV^T += dO^T P; role 1 holds V^T and forms dP = dO V^T, reads the
// bf16 P its partner left in LDS, forms dS = P (dP - D) and
// dK^T += Q^T dS.  With one resident operand and one accumulator per wave
// (~210 registers at d = 128 with the deferred products' state; both
// operands and accumulators on one wave would need ~350), eight waves -- two
// per SIMD -- share a 128-key workgroup.  Waves w and w + 4 (one SIMD) form
// pair w.  Per 32-query block the pair meets at one barrier (P handed over);
// between two barriers role 0 forms S and P of block b while its dV^T update
// for block b - 1 runs on the matrix cores, and role 1 forms dP of block b
// while it computes dS of block b - 1, then adds block b - 1 into dK^T.
// LSE and D enter as the starting values of the S and dP accumulators
// (-LSE/scale and -D, from the workspace as the first kernel stored them),
// so P = exp2(c s) and dS = P s without a per-element correction.  Q and dO rows are read row-wise for the first product and
// through ds_read_b64_tr_b16 for the second.
template <int D, int BQ, bool CAUSAL, bool F16, bool PACKED, int PD = 3>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512)))
void fa_bwd_dkdv_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                             const bf16* __restrict__ v, const bf16* __restrict__ dout,
                             const float* __restrict__ nlse, const float* __restrict__ ndsum,
                             bf16* __restrict__ dk, bf16* __restrict__ dv, int BH, BwdLayout lay,
                             float c /* scale*log2(e) */, float scale) {
  constexpr int NW = 8, NP = NW / 2;
  constexpr int RB = D * 2;
  constexpr int BC = NP * 32;           // keys per workgroup
  constexpr int TILE = BQ * RB;         // bytes of one Q (or dO) tile
  constexpr int STAGE = 2 * TILE + 2 * BQ * 4;
  constexpr int PBLK = 32 * 32 * 2;     // one pair's bf16 P block
  constexpr int NB = BQ / 32;           // 32-query blocks per tile
  constexpr int NC = D / 32, NF1 = D / 16, NF2 = 2 * NC;
  // steps of the loops that interleave one product with the other role's
  // eight pairs of exponentials (or dS values): at least eight
  constexpr int NS1 = NF1 + PD > 8 ? NF1 + PD : 8, NS2 = NF2 + PD > 8 ? NF2 + PD : 8;
  static_assert(BQ % 64 == 0 && NB % 2 == 0, "query tile of an even number of 32-row blocks");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE + 2 * NP * PBLK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave / NP, pair = wave % NP;
  const int l32 = lane & 31, g = lane >> 5;
  const int bh = blockIdx.x % BH;
  const int kt = blockIdx.x / BH;       // heaviest (earliest keys) first under causal
  const BwdSeq sq = bwd_seq<D, PACKED>(lay, bh);
  const int Lq = sq.Lq, Lk = sq.Lk;
  const int rs = PACKED ? sq.rs : D;    // row stride in elements (a constant when dense)
  const int k0 = kt * BC;
  if (k0 >= Lk) return;                 // past this sequence's keys (whole workgroup)
  const int off = CAUSAL ? Lk - Lq : 0; // causal: query i sees keys j <= i + off
  const int kw = k0 + pair * 32;        // the pair's first key
  const int my_key = kw + l32;

  const uint32_t RG = (uint32_t)rs * 2u;       // bytes from one row to the next in memory
  const rsrc_t Qr = make_rsrc(q + sq.qbase, (uint32_t)Lq * RG);
  const rsrc_t Or = make_rsrc(dout + sq.qbase, (uint32_t)Lq * RG);
  const rsrc_t Lr = make_rsrc(nlse + sq.lbase, (uint32_t)Lq * 4u);
  const rsrc_t Dr = make_rsrc(ndsum + sq.lbase, (uint32_t)Lq * 4u);

  bf16x8 kv[D / 16];
  {
    const rsrc_t R = make_rsrc((role ? v : k) + sq.kbase, (uint32_t)Lk * RG);
#pragma unroll
    for (int u = 0; u < D / 16; ++u)
      kv[u] = __builtin_bit_cast(bf16x8, buf_load16(R, (uint32_t)my_key * RG + (16u * u + 8u * g) * 2u));
  }

  TileLoader<RB, BQ, NW> ld;
  ld.init(wave, lane, RG);
  TileReads<D> rd;
  rd.init(lane);

  const int nqt = (Lq + BQ - 1) / BQ;
  // the first query tile that sees one of this workgroup's keys
  const int it0 = CAUSAL ? max(k0 - off, 0) / BQ : 0;
  auto load_tile = [&](int it) {
    uint8_t* st = smem + (it & 1) * STAGE;
    const uint32_t qoff = (uint32_t)it * BQ * RG;
    ld.load(Qr, qoff, st, wave);
    ld.load(Or, qoff, st + TILE, wave);
    if (wave < 2 * (BQ / 64)) {           // -LSE/scale (even waves) and -D (odd), 64 rows each
      const int which = wave & 1, part = wave >> 1;
      const uint32_t off = ((uint32_t)it * BQ + 64 * part + lane) * 4u;
      lds_dma4(which ? Dr : Lr, st + 2 * TILE + which * BQ * 4 + 64 * part * 4, off);
    }
  };

  f32x16 acc[NC];                       // dV^T (role 0) or dK^T (role 1)
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) acc[cb] = f32x16{};

  if (it0 < nqt) load_tile(it0);
  wait_vm();                            // also completes the K^T / V^T loads above
  __syncthreads();

  // The second product of each 32-query block (dV^T += dO^T P on role 0,
  // dK^T += Q^T dS on role 1) is deferred to the next block's interval, where
  // it runs beside that block's exponentials (role 0) or beside its
  // dP MFMAs (role 1), instead of after a barrier with nothing to overlap.
  // Every interval has the same shape: the workgroup's first interval defers
  // products of zero P and dS, and blocks wholly before the pair's keys
  // (causal) are computed and masked to zero like the diagonal blocks.  Each
  // role runs its own copy of the loop (the same barriers in the same order),
  // so each keeps only its own state live.
  // P slots start at zero (the first interval's deferred dS reads one)
  *reinterpret_cast<u32x4*>(smem + 2 * STAGE + tid * 16) = u32x4{0u, 0u, 0u, 0u};
  *reinterpret_cast<u32x4*>(smem + 2 * STAGE + 8192 + tid * 16) = u32x4{0u, 0u, 0u, 0u};
  static_assert(2 * NP * PBLK == 2 * 8192 && NW * 64 * 16 == 8192, "P slots cleared by one pass");
  __syncthreads();

  auto run = [&](auto ROLE) __attribute__((always_inline)) {
    constexpr int R = decltype(ROLE)::value;
    // the deferred block's transposed operand (the first tile's, for the
    // first interval's zero products)
    const uint8_t* pA2 = smem + (it0 & 1) * STAGE + (R ? 0 : TILE);
    [[maybe_unused]] const uint8_t* ppb = smem + 2 * STAGE + (NP + pair) * PBLK;   // its P slot
    int pr0 = 0;                        // its first row within the tile
    [[maybe_unused]] bf16x8 pbo[2] = {};   // role 0: its P as B operands
    [[maybe_unused]] f32x16 ps = f32x16{};   // role 1: its dP - D

    auto second = [&](const bf16x8 (&bo)[2]) __attribute__((always_inline)) {
      bf16x8 f[NF2];
#pragma unroll
      for (int i = 0; i < NF2 + PD; ++i) {
        if (i < NF2) f[i] = rd.trfrag(pA2, pr0 + 16 * (i / NC), i % NC);
        if (i >= PD) {
          const int x = i - PD;
          acc[x % NC] = mma16<F16>(f[x], bo[x / NC], acc[x % NC]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // role 1: dS of the deferred block, pair h, from its P (LDS) and dP - D
    auto ds_pair = [&](const u32x4& lo, const u32x4& hi, int h) __attribute__((always_inline)) {
      const int i = 2 * h;
      const uint32_t w = h < 4 ? lo[h] : hi[h - 4];
      return pack16<F16>(lo16<F16>(w) * ps[i], hi16<F16>(w) * ps[i + 1]);
    };

    for (int it = it0; it < nqt; ++it) {
      const uint8_t* st = smem + (it & 1) * STAGE;
      const uint8_t* Qs = st;
      const uint8_t* Os = st + TILE;
      const float* Ls = reinterpret_cast<const float*>(st + 2 * TILE);
      const float* Ds = Ls + BQ;

#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const int qb0 = it * BQ + 32 * blk;
        uint8_t* pb = smem + 2 * STAGE + ((blk & 1) * NP + pair) * PBLK;
        if constexpr (R == 0) {
          const bool edge = (CAUSAL && qb0 + off < kw + 31) || qb0 + 32 > Lq;
          // ---- S - LSE/scale for this block (the accumulator starts at
          // -LSE/scale, so exp2(c * s) is P) ----
          f32x16 s;
#pragma unroll
          for (int gi = 0; gi < 4; ++gi) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(Ls + 32 * blk + 8 * gi + 4 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j) s[4 * gi + j] = x[j];
          }
          {
            bf16x8 f[NF1];
#pragma unroll
            for (int i = 0; i < NF1 + PD; ++i) {
              if (i < NF1) f[i] = rd.rowfrag(Qs, 32 * blk, i);
              if (i >= PD) s = mma16<F16>(f[i - PD], kv[i - PD], s);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          // masked scores to -inf, so that their weights come out as 0
          if (edge) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int qi = qb0 + 8 * (e >> 2) + 4 * g + (e & 3);
              if (qi >= Lq || (CAUSAL && my_key > qi + off)) s[e] = -__builtin_inff();
            }
          }
          // ---- P of this block, beside dV^T += dO^T P of the deferred block ----
          uint32_t pw[8];
          {
            bf16x8 f[NF2];
#pragma unroll
            for (int i = 0; i < NS2; ++i) {
              if (i < NF2) f[i] = rd.trfrag(pA2, pr0 + 16 * (i / NC), i % NC);
              if (i >= PD && i < NF2 + PD) {
                const int x = i - PD;
                acc[x % NC] = mma16<F16>(f[x], pbo[x / NC], acc[x % NC]);
              }
              if (i < 8) {
                const int e = 2 * i;
                const float p0 = __builtin_amdgcn_exp2f(s[e] * c);
                const float p1 = __builtin_amdgcn_exp2f(s[e + 1] * c);
                pw[i] = pack16<F16>(p0, p1);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          *reinterpret_cast<u32x4*>(pb + 16 * lane) = u32x4{pw[0], pw[1], pw[2], pw[3]};
          *reinterpret_cast<u32x4*>(pb + 1024 + 16 * lane) = u32x4{pw[4], pw[5], pw[6], pw[7]};
          pbo[0] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
          pbo[1] = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});
          pA2 = Os;
        } else {
          // ---- dP - D for this block (the accumulator starts at -D), beside
          // dS of the deferred block ----
          const u32x4 plo = *reinterpret_cast<const u32x4*>(ppb + 16 * lane);
          const u32x4 phi = *reinterpret_cast<const u32x4*>(ppb + 1024 + 16 * lane);
          f32x16 s;
#pragma unroll
          for (int gi = 0; gi < 4; ++gi) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(Ds + 32 * blk + 8 * gi + 4 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j) s[4 * gi + j] = x[j];
          }
          uint32_t sw[8];
          {
            bf16x8 f[NF1];
#pragma unroll
            for (int i = 0; i < NS1; ++i) {
              if (i < NF1) f[i] = rd.rowfrag(Os, 32 * blk, i);
              if (i >= PD && i < NF1 + PD) s = mma16<F16>(f[i - PD], kv[i - PD], s);
              if (i < 8) sw[i] = ds_pair(plo, phi, i);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          // ---- dK^T += Q^T dS of the deferred block ----
          const bf16x8 bo[2] = {__builtin_bit_cast(bf16x8, u32x4{sw[0], sw[1], sw[2], sw[3]}),
                                __builtin_bit_cast(bf16x8, u32x4{sw[4], sw[5], sw[6], sw[7]})};
          second(bo);
          ps = s;
          pA2 = Qs;
          ppb = pb;
        }
        lds_barrier();                  // this block's P is in LDS
        // the previous tile's stage is free once every wave is past the first
        // block's interval (its last block was deferred into it)
        if (blk == 0 && it + 1 < nqt) load_tile(it + 1);
        pr0 = 32 * blk;
      }

      if (it + 1 < nqt) wait_vm();
      __syncthreads();
    }

    // ---- the last block's deferred second product (none without a query
    // tile: then dK and dV stay zero) ----
    if (it0 >= nqt) return;
    if constexpr (R == 0) {
      second(pbo);
    } else {
      const u32x4 plo = *reinterpret_cast<const u32x4*>(ppb + 16 * lane);
      const u32x4 phi = *reinterpret_cast<const u32x4*>(ppb + 1024 + 16 * lane);
      uint32_t sw[8];
#pragma unroll
      for (int h = 0; h < 8; ++h) sw[h] = ds_pair(plo, phi, h);
      const bf16x8 bo[2] = {__builtin_bit_cast(bf16x8, u32x4{sw[0], sw[1], sw[2], sw[3]}),
                            __builtin_bit_cast(bf16x8, u32x4{sw[4], sw[5], sw[6], sw[7]})};
      second(bo);
    }
  };
  if (role == 0) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});
  __syncthreads();                      // every wave is done with the tile buffers

  // ---- epilogue: lane holds key my_key, features 32cb + 8(i/4) + 4g + i%4;
  // whole rows of dV (role 0) or dK (role 1) through LDS, 32 rows per wave ----
  static_assert(NW * 32 * RB <= (int)sizeof(smem), "output staging fits the tile buffers");
  bf16* out = (role ? dk : dv) + sq.kbase;
  store_tile_rows<F16, D>(smem + wave * 32 * RB, acc, role ? scale : 1.f, lane, Lk - kw,
                          [&](int r) { return out + (size_t)(kw + r) * rs; });
}

// ---------------------------------------------------------------------------
// 3. dQ: query tiles outer
// ---------------------------------------------------------------------------
template <int D, int BC, int NW, bool CAUSAL, bool F16, bool PACKED>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
void fa_bwd_dq_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                      const bf16* __restrict__ v, const bf16* __restrict__ dout,
                      const float* __restrict__ lse, const float* __restrict__ ndsum,
                      bf16* __restrict__ dq, int BH, BwdLayout lay, float c, float scale) {
  constexpr int RB = D * 2;
  constexpr int BR = NW * 32;           // queries per workgroup
  constexpr int TILE = BC * RB;
  constexpr int STAGE = 2 * TILE;
  constexpr float kLog2e = 1.44269504088896340736f;
  static_assert(BC % 32 == 0, "key tile of whole 32-key blocks");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the block skips are scalar branches
  const int l32 = lane & 31, g = lane >> 5;
  const int bh = blockIdx.x % BH;
  const BwdSeq sq = bwd_seq<D, PACKED>(lay, bh);
  const int Lq = sq.Lq, Lk = sq.Lk;
  const int rs = PACKED ? sq.rs : D;         // row stride in elements (a constant when dense)
  const int nqt = (Lq + BR - 1) / BR;
  int qt = blockIdx.x / BH;
  if (qt >= nqt) return;                     // past this sequence's queries (whole workgroup)
  if constexpr (CAUSAL) qt = nqt - 1 - qt;   // longest query tiles first
  const int off = CAUSAL ? Lk - Lq : 0;      // causal: query i sees keys j <= i + off
  const int q0 = qt * BR;
  const int qw = q0 + wave * 32;
  const int my_q = qw + l32;

  const uint32_t RG = (uint32_t)rs * 2u;     // bytes from one row to the next in memory
  const rsrc_t Kr = make_rsrc(k + sq.kbase, (uint32_t)Lk * RG);
  const rsrc_t Vr = make_rsrc(v + sq.kbase, (uint32_t)Lk * RG);

  // Q^T and dO^T of this lane's query as B operands; its LSE (base 2) and -D
  bf16x8 qb[D / 16], ob[D / 16];
  float lse2 = 0.f, nd = 0.f;
  {
    const rsrc_t Qr = make_rsrc(q + sq.qbase, (uint32_t)Lq * RG);
    const rsrc_t Or = make_rsrc(dout + sq.qbase, (uint32_t)Lq * RG);
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      const uint32_t o16 = (uint32_t)my_q * RG + (16u * u + 8u * g) * 2u;
      qb[u] = __builtin_bit_cast(bf16x8, buf_load16(Qr, o16));
      ob[u] = __builtin_bit_cast(bf16x8, buf_load16(Or, o16));
    }
    if (my_q < Lq) {
      // a query that sees no key has LSE = -inf; +inf here makes every one of
      // its weights exp2(-inf) = 0, masked or not
      const float l = lse[sq.lbase + my_q];
      lse2 = l > -__builtin_inff() ? l * kLog2e : __builtin_inff();
      nd = ndsum[sq.lbase + my_q];
    }
  }

  TileLoader<RB, BC, NW> ld;
  ld.init(wave, lane, RG);
  TileReads<D> rd;
  rd.init(lane);

  const int kv_end = CAUSAL ? min(Lk, max(q0 + BR + off, 0)) : Lk;
  const int ntiles = (kv_end + BC - 1) / BC;
  auto load_tile = [&](int j) {
    uint8_t* st = smem + (j & 1) * STAGE;
    const uint32_t off = (uint32_t)j * BC * RG;
    ld.load(Kr, off, st, wave);
    ld.load(Vr, off, st + TILE, wave);
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};

  load_tile(0);
  wait_vm();
  __syncthreads();

  // every dP^T block of this lane starts at its query's -D (16 registers
  // held across the loop; the first MFMA of each chain reads them as C)
  f32x16 ndv;
#pragma unroll
  for (int i = 0; i < 16; ++i) ndv[i] = nd;

  for (int j = 0; j < ntiles; ++j) {
    const bool more = j + 1 < ntiles;
    if (more) load_tile(j + 1);
    const uint8_t* Ks = smem + (j & 1) * STAGE;
    const uint8_t* Vs = Ks + TILE;

#pragma unroll
    for (int blk = 0; blk < BC / 32; ++blk) {
      const int kb0 = j * BC + 32 * blk;
      // the wave is past its sequence's queries, or the block lies above the diagonal
      if (qw >= Lq || (CAUSAL && kb0 > qw + 31 + off)) continue;
      // ---- S^T = K Q^T and dP^T = V dO^T: keys on rows, this lane's query on the column ----
      // dP^T starts at -D (the lane's query), so dS = P dp
      f32x16 s = f32x16{}, dp = ndv;
      {
        constexpr int PD = 4, NF = 2 * (D / 16);
        bf16x8 f[NF];
#pragma unroll
        for (int i = 0; i < NF + PD; ++i) {
          if (i < NF) f[i] = rd.rowfrag((i & 1) ? Vs : Ks, 32 * blk, i >> 1);
          if (i >= PD) {
            const int x = i - PD;
            if (x & 1) dp = mma16<F16>(f[x], ob[x >> 1], dp);
            else s = mma16<F16>(f[x], qb[x >> 1], s);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // ---- dS^T (row i of the accumulator is key kb0 + 8(i/4) + 4g + i%4) ----
      // (one comparison for both lengths: with separate ones the compiler's
      // register allocation of this loop spills)
      const bool edge = (CAUSAL && kb0 + 31 > qw + off) || max(kb0 + 32 - Lk, qw + 32 - Lq) > 0;
      // masked scores to -inf, so that their weights come out as 0
      if (edge) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb0 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key >= Lk || my_q >= Lq || (CAUSAL && key > my_q + off)) s[i] = -__builtin_inff();
        }
      }
      bf16x8 ps[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint32_t w[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          float dsv[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int i = 8 * t + 2 * h + e;
            const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c, -lse2));
            dsv[e] = p * dp[i];
          }
          w[h] = pack16<F16>(dsv[0], dsv[1]);
        }
        ps[t] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
      }
      // ---- dQ^T += K^T dS^T ----
      {
        constexpr int PD = 4, NC = D / 32, NF = 2 * NC;
        bf16x8 f[NF];
#pragma unroll
        for (int i = 0; i < NF + PD; ++i) {
          if (i < NF) f[i] = rd.trfrag(Ks, 32 * blk + 16 * (i / NC), i % NC);
          if (i >= PD) {
            const int x = i - PD;
            acc[x % NC] = mma16<F16>(f[x], ps[x / NC], acc[x % NC]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    if (more) wait_vm();
    __syncthreads();
  }

  // whole dQ rows through LDS, 32 rows per wave
  static_assert(NW * 32 * RB <= (int)sizeof(smem), "output staging fits the tile buffers");
  store_tile_rows<F16, D>(smem + wave * 32 * RB, acc, scale, lane, Lq - qw,
                          [&](int r) { return dq + sq.qbase + (size_t)(qw + r) * rs; });
}

// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool F16, bool PACKED>
static hipError_t launch_bwd_d(const BwdArgs& a) {
  // dK/dV: 128 keys per workgroup (four wave pairs, two waves per SIMD),
  // 128-query tiles (against 64: +3% at N = 16384, causal).
  // dQ: 256 queries per workgroup, 128-key tiles (measured against 32- and
  // 64-key tiles in one process).
  constexpr int BQ = 128, NWK = 8, BCK = NWK / 2 * 32;   // BCK keys per dK/dV workgroup
  constexpr int BCQ = 128, NWQ = 8;
  const int BH = a.B * a.H;
  hipStream_t st = (hipStream_t)a.stream;
  const bool packed = PACKED;
  const BwdLayout lay{a.cu_q, a.cu_k, a.H, a.N, packed ? a.Nk : a.N, a.total_q, a.total_k};
  // -D and -LSE/scale for every query row: B*H*N dense rows, or total_q*H
  // packed rows
  const long long rows = packed ? (long long)a.total_q * a.H : (long long)BH * a.N;
  hipLaunchKernelGGL((fa_bwd_pre_kernel<D, F16>), dim3((unsigned)((rows + (256 / (D / 8)) - 1) / (256 / (D / 8)))),
                     dim3(256), 0, st, (const bf16*)a.o, (const bf16*)a.dout, a.lse, a.ndsum, a.nlse,
                     rows, packed ? a.H : 0, a.total_q, -1.f / a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkt = (lay.Nk + BCK - 1) / BCK;   // of the longest key sequence
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, BQ, CAUSAL, F16, PACKED>), dim3((unsigned)((long long)nkt * BH)),
                     dim3(NWK * 64), 0, st, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
                     (const bf16*)a.dout, a.nlse, a.ndsum, (bf16*)a.dk, (bf16*)a.dv, BH, lay,
                     a.scale_log2, a.scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqt = (a.N + NWQ * 32 - 1) / (NWQ * 32);   // of the longest query sequence
  hipLaunchKernelGGL((fa_bwd_dq_kernel<D, BCQ, NWQ, CAUSAL, F16, PACKED>), dim3((unsigned)((long long)nqt * BH)),
                     dim3(NWQ * 64), 0, st, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
                     (const bf16*)a.dout, a.lse, a.ndsum, (bf16*)a.dq, BH, lay, a.scale_log2,
                     a.scale);
  return hipGetLastError();
}

template <bool F16, bool PACKED>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  if (a.d == 128)
    return a.causal ? launch_bwd_d<128, true, F16, PACKED>(a) : launch_bwd_d<128, false, F16, PACKED>(a);
  return a.causal ? launch_bwd_d<64, true, F16, PACKED>(a) : launch_bwd_d<64, false, F16, PACKED>(a);
}

hipError_t launch_bwd(const BwdArgs& a) {
  if (a.cu_q) {   // packed sequences: bf16 only
    if (a.in_f16) return hipErrorNotSupported;
    return launch_bwd_t<false, true>(a);
  }
  return a.in_f16 ? launch_bwd_t<true, false>(a) : launch_bwd_t<false, false>(a);
}

}  // namespace fa
