// bf16 -> block-scaled fp8 (E4M3FN) quantisation of Q, K or V, with the
// optional incoherent processing of Q and K.
//
// Method: the FlashAttention-3 snippets pair block quantisation with
// "incoherent processing" to cut fp8 error.  Block quantisation here is the
// fp8 forward pass's input format: per (batch, head) and 64-row block,
// scale = max|x| / 448, or the smallest power of two with max|x| / scale <=
// 448 (1 for an all-zero block either way), and code = E4M3FN(x / scale),
// nearest with ties to even.  Incoherent processing is read as the
// multiplication of each row by diag(s) H_d / sqrt(d) -- random signs s, the
// Sylvester-ordered Walsh-Hadamard matrix H_d -- before the scale is taken;
// applied to Q and K with the same s it leaves Q K^T unchanged while
// spreading a large entry over all d coordinates.
//
// gfx950 mapping: a memory-bound pass (2 bytes read, 1 written per element).
// A workgroup is one 64-row scale block of one (batch, head) and two waves,
// 32 rows each; the block maximum is a wave reduction plus one exchange
// through LDS, and many small workgroups per CU overlap their loads with
// each other's arithmetic.  The rows arrive in LDS by direct global->LDS
// loads, their 16-byte chunks XOR-swizzled by the row index so that the
// fragment reads below hit distinct banks.  Each lane reads its row's
// 16-byte chunks as the B operand of a 32x32x16 MFMA (row 32w + lane%32,
// 8 consecutive columns per 16-column step).
//  * Rotated blocks run the rotation on the matrix cores as the product
//    Y^T = (diag(s) H_d)^T X^T: every entry of diag(s) H_d is +-1, exact in
//    bf16, and the products of bf16 inputs with it are exact, so only the
//    fp32 accumulation rounds (as a d-point butterfly network would).  The
//    +-1 fragments are made in registers: the sign of H_d[k][j] is the
//    parity of popcount(k & j), which splits into a per-lane pattern over
//    the 8 consecutive k of a fragment, a per-lane bit per 16-k step and a
//    bit fixed by the 32-column block; the random signs s flip the sign bits
//    of the X fragments.  A lane then holds four consecutive output columns
//    of one row per accumulator group.
//  * Plain blocks quantise the fragments as read: eight consecutive columns
//    of one row per 16-column step.
// The 1/sqrt(d) factor is folded into the block's reciprocal scale, and each
// ratio x * (448 / max|x|) (within an ulp or so of x / scale), or x * 2^-k
// for a power-of-two scale 2^k (exact), is clamped to +-448 and converted by
// v_cvt_pk_fp8_f32 (nearest, ties to even).  The
// codes go back through LDS, four to a 32-bit word, so that every store
// instruction writes 1 KB of consecutive rows.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

template <int D, bool ROT>
__global__ __attribute__((amdgpu_flat_work_group_size(128, 128)))
__attribute__((amdgpu_waves_per_eu(3)))
void fa_fp8_quant_kernel(const bf16* __restrict__ x, const float* __restrict__ signs,
                             uint8_t* __restrict__ codes, float* __restrict__ scales, int N,
                             int rtiles, int pow2) {
  constexpr int RB = D * 2;             // bytes per bf16 row
  constexpr int NCH = RB / 16;          // 16-byte chunks per row
  constexpr int ROWS = 64;              // one scale block, 32 rows per wave
  [[maybe_unused]] constexpr int NI = ROWS * RB / 1024;  // 1 KB direct-load instructions per block
  constexpr int NKS = D / 16;           // 16-k steps of the product
  constexpr int NCB = D / 32;           // 32-column blocks of Y
  static_assert(D == 64 || D == 128, "d of 64 or 128");
  __shared__ __attribute__((aligned(16))) uint8_t tile[ROWS * RB];
  __shared__ float wmax[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int bh = blockIdx.x / rtiles, rt = blockIdx.x % rtiles;
  const int r0 = rt * ROWS;
  const size_t head = (size_t)bh * (size_t)N * D;
  const int rows_here = min(ROWS, N - r0);
  [[maybe_unused]] const rsrc_t Xr = make_rsrc(x + head + (size_t)r0 * D, (uint32_t)rows_here * RB);

#if defined(__HIP_DEVICE_COMPILE__)  // the LDS-DMA builtin exists in the device pass only
#pragma unroll
  for (int x2 = 0; x2 < NI / 2; ++x2) {
    const int i = wave * (NI / 2) + x2;
    const int byte = i * 1024 + lane * 16;
    const int r = byte / RB, p = (byte % RB) / 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        Xr, (__attribute__((address_space(3))) void*)(tile + i * 1024), 16,
        (uint32_t)(r * RB + 16 * (p ^ (r % NCH))), 0, 0, 0);
  }
#endif

  // sign bits of s for this lane's k = 16 ks + 8 g + e (e = 0..7), as XOR
  // masks over bf16 pairs
  uint32_t smask[NKS][4] = {};
#pragma unroll
  for (int ks = 0; ks < NKS && ROT; ++ks) {
    const float* sk = signs + 16 * ks + 8 * g;   // 4-byte aligned: scalar loads
#pragma unroll
    for (int w = 0; w < 4; ++w)
      smask[ks][w] = ((as_u32(sk[2 * w]) >> 16) & 0x8000u) | (as_u32(sk[2 * w + 1]) & 0x80000000u);
  }
  // H_d fragment pattern: (-1)^popcount((l32 + 32 cb) & (16 ks + 8 g + e))
  //   = (-1)^popcount(l32 & e) * (-1)^popcount(l32 & (16 ks + 8 g) & 31) * (-1)^popcount(cb & (ks / 2))
  uint32_t hpat[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = (__builtin_popcount(l32 & (2 * w)) & 1) ? 0xBF80u : 0x3F80u;
    const uint32_t hi = (__builtin_popcount(l32 & (2 * w + 1)) & 1) ? 0xBF80u : 0x3F80u;
    hpat[w] = lo | (hi << 16);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's share has landed
  __syncthreads();

  // X^T fragments of this wave's 32 rows with the signs applied: row
  // 32 wave + l32, k = 16 ks + 8 g .. + 7 (one 16-byte chunk)
  const int r = 32 * wave + l32;
  bf16x8 xf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    u32x4 w4 = *reinterpret_cast<const u32x4*>(tile + r * RB + 16 * ((2 * ks + g) ^ (r % NCH)));
#pragma unroll
    for (int w = 0; w < 4; ++w) w4[w] ^= smask[ks][w];
    xf[ks] = __builtin_bit_cast(bf16x8, w4);
  }
  // ROT: Y^T = (diag(s) H_d)^T X^T; lane: output columns 32 cb + 8 qg + 4 g
  // .. + 3 of row r in acc[cb][4 qg .. 4 qg + 3].  Plain: the fragments
  // themselves, lane: columns 16 ks + 8 g .. + 7 of row r.
  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x16{};
  if constexpr (ROT) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint32_t lb = (__builtin_popcount(l32 & ((16 * ks + 8 * g) & 31)) & 1) ? 0x80008000u : 0u;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const uint32_t f = lb ^ ((__builtin_popcount(cb & (ks >> 1)) & 1) ? 0x80008000u : 0u);
        const bf16x8 hf = __builtin_bit_cast(bf16x8, u32x4{hpat[0] ^ f, hpat[1] ^ f, hpat[2] ^ f, hpat[3] ^ f});
        acc[cb] = mfma32x32x16(hf, xf[ks], acc[cb]);
      }
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const u32x4 w4 = __builtin_bit_cast(u32x4, xf[ks]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc[ks / 2][8 * (ks & 1) + 2 * w] = bf16lo(w4[w]);
        acc[ks / 2][8 * (ks & 1) + 2 * w + 1] = bf16hi(w4[w]);
      }
    }
  }

  // the block: amax (both waves), scale, and the reciprocal factor taking y
  // to x / scale
  // (rotated rows still lack the factor 1/sqrt(d); it is applied here)
  constexpr float fct = ROT ? (D == 64 ? 0.125f : 0.08838834764831845f) : 1.f;
  float amax = 0.f;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(acc[cb][i]));   // rows past N are 0
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();                      // wmax is set and every X fragment has been read
  amax = fmaxf(wmax[0], wmax[1]) * fct;
  float scale = amax > 0.f ? amax / 448.f : 1.f;
  float rinv = amax > 0.f ? fct * (448.f / amax) : 0.f;
  if (pow2 && amax > 0.f) {
    // amax = f 2^e, f in [0.5, 1), 448 = 0.875 2^9: the smallest 2^k with
    // amax <= 448 2^k has k = e - 9 for f <= 0.875, else e - 8
    const int e = __builtin_amdgcn_frexp_expf(amax);
    const int kk = __builtin_amdgcn_frexp_mantf(amax) <= 0.875f ? e - 9 : e - 8;
    scale = __builtin_amdgcn_ldexpf(1.f, kk);
    rinv = __builtin_amdgcn_ldexpf(fct, -kk);
  }
  if (tid == 0) scales[(size_t)bh * ((N + 63) >> 6) + rt] = scale;

  // codes: four consecutive columns of row r per 32-bit word, into LDS with
  // the 16-byte chunks of each row swizzled by the row
  constexpr int CB = D;                 // code bytes per row
  constexpr int CCH = CB / 16;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int qg = 0; qg < 4; ++qg) {
      float t[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        t[u] = fminf(fmaxf(acc[cb][4 * qg + u] * rinv, -448.f), 448.f);
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], pk, true);
      // ROT: columns 32 cb + 8 qg + 4 g; plain: 16 ks + 8 g + 4 (qg & 1), ks = 2 cb + qg / 2
      const int col = ROT ? 32 * cb + 8 * qg + 4 * g : 16 * (2 * cb + qg / 2) + 8 * g + 4 * (qg & 1);
      *reinterpret_cast<uint32_t*>(tile + r * CB + 16 * ((col >> 4) ^ (r % CCH)) + (col & 15)) = (uint32_t)pk;
    }
  __syncthreads();
  uint8_t* out = codes + head + (size_t)r0 * D;
#pragma unroll
  for (int x2 = 0; x2 < ROWS * CB / 2048; ++x2) {
    const int i = wave * (ROWS * CB / 2048) + x2;
    const int byte = i * 1024 + lane * 16;
    const int row = byte / CB, c = (byte % CB) / 16;
    if (row < rows_here)
      *reinterpret_cast<u32x4*>(out + byte) =
          *reinterpret_cast<const u32x4*>(tile + row * CB + 16 * (c ^ (row % CCH)));
  }
}

template <int D>
static hipError_t launch_quant_d(const QuantArgs& a) {
  const int rtiles = (a.N + 63) / 64;
  const long long grid = (long long)a.B * a.H * rtiles;
  hipStream_t st = (hipStream_t)a.stream;
  if (a.signs)
    hipLaunchKernelGGL((fa_fp8_quant_kernel<D, true>), dim3((unsigned)grid), dim3(128), 0, st,
                       (const bf16*)a.x, a.signs, (uint8_t*)a.codes, a.scales, a.N, rtiles, a.pow2);
  else
    hipLaunchKernelGGL((fa_fp8_quant_kernel<D, false>), dim3((unsigned)grid), dim3(128), 0, st,
                       (const bf16*)a.x, a.signs, (uint8_t*)a.codes, a.scales, a.N, rtiles, a.pow2);
  return hipGetLastError();
}

hipError_t launch_fp8_quant(const QuantArgs& a) {
  return a.d == 128 ? launch_quant_d<128>(a) : launch_quant_d<64>(a);
}

}  // namespace fa
