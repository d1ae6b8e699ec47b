// bf16 -> block-scaled fp8 (E4M3FN) quantisation of Q, K or V, with the
// optional incoherent processing of Q and K.
//
// Method: the FlashAttention-3 snippets pair block quantisation with
// "incoherent processing" to cut fp8 error.  Block quantisation here is the
// fp8 forward pass's input format: per (batch, head) and 64-row block,
// scale = max|x| / 448 (1 for an all-zero block) and code = E4M3FN(x /
// scale), nearest with ties to even.  Incoherent processing is read as the
// multiplication of each row by diag(s) H_d / sqrt(d) -- random signs s, the
// Sylvester-ordered Walsh-Hadamard matrix H_d -- before the scale is taken;
// applied to Q and K with the same s it leaves Q K^T unchanged while
// spreading a large entry over all d coordinates.
//
// gfx950 mapping: a memory-bound pass (2 bytes read, 1 written per element).
// A workgroup is one wave and one 64-row scale block of one (batch, head),
// so the block maximum is a wave reduction and many small workgroups per CU
// overlap their loads with each other's arithmetic.  The rows arrive in LDS
// by direct global->LDS loads, their 16-byte chunks XOR-swizzled by the row
// index so that the row-per-thread reads below hit distinct banks.  Each
// thread then owns one row: bf16 -> fp32, signs, the d-point fast
// Walsh-Hadamard transform in registers (log2 d butterfly stages).  The
// 1/sqrt(d) factor is folded into the block's reciprocal scale, and each
// ratio x * (448 / max|x|) (within an ulp or so of x / scale) is clamped to
// +-448 and converted by v_cvt_pk_fp8_f32 (nearest, ties to even).  The
// codes go back through LDS so that every store instruction writes 1 KB of
// consecutive rows.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

template <int D, bool ROT>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64)))
void fa_fp8_quant_kernel(const bf16* __restrict__ x, const float* __restrict__ signs,
                         uint8_t* __restrict__ codes, float* __restrict__ scales, int N,
                         int rtiles) {
  constexpr int RB = D * 2;             // bytes per bf16 row
  constexpr int NCH = RB / 16;          // 16-byte chunks per row
  constexpr int ROWS = 64;              // one scale block
  [[maybe_unused]] constexpr int NI = ROWS * RB / 1024;  // 1 KB direct-load instructions per block
  static_assert(D == 64 || D == 128, "d of 64 or 128");
  __shared__ __attribute__((aligned(16))) uint8_t tile[ROWS * RB];
  __shared__ float sg[D];

  const int tid = threadIdx.x, lane = tid;
  const int bh = blockIdx.x / rtiles, rt = blockIdx.x % rtiles;
  const int r0 = rt * ROWS;
  const size_t head = (size_t)bh * (size_t)N * D;
  const int rows_here = min(ROWS, N - r0);
  [[maybe_unused]] const rsrc_t Xr = make_rsrc(x + head + (size_t)r0 * D, (uint32_t)rows_here * RB);

#if defined(__HIP_DEVICE_COMPILE__)  // the LDS-DMA builtin exists in the device pass only
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int blk = i;
    const int byte = blk * 1024 + lane * 16;
    const int r = byte / RB, p = (byte % RB) / 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        Xr, (__attribute__((address_space(3))) void*)(tile + blk * 1024), 16,
        (uint32_t)(r * RB + 16 * (p ^ (r % NCH))), 0, 0, 0);
  }
#endif
  if (ROT)
    for (int i = tid; i < D; i += 64) sg[i] = signs[i];
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the loads have landed
  __syncthreads();

  // this thread's row, fp32
  const int r = tid;
  float v[D];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(tile + r * RB + 16 * (c ^ (r % NCH)));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * c + 2 * e] = bf16lo(w[e]);
      v[8 * c + 2 * e + 1] = bf16hi(w[e]);
    }
  }
  if constexpr (ROT) {
#pragma unroll
    for (int i = 0; i < D; ++i) v[i] *= sg[i];
    // y = H_d v in Sylvester order: butterflies (a, b) -> (a + b, a - b)
#pragma unroll
    for (int len = 1; len < D; len <<= 1)
#pragma unroll
      for (int i = 0; i < D; i += 2 * len)
#pragma unroll
        for (int j = i; j < i + len; ++j) {
          const float a = v[j], b = v[j + len];
          v[j] = a + b;
          v[j + len] = a - b;
        }
  }
  // (rotated rows still lack the factor 1/sqrt(d); it is applied below)
  constexpr float f = ROT ? (D == 64 ? 0.125f : 0.08838834764831845f) : 1.f;

  // the block: amax, scale, and the reciprocal factor taking v to x / scale
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < D; ++i) amax = fmaxf(amax, fabsf(v[i]));   // rows past N are 0
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  amax *= f;
  const float scale = amax > 0.f ? amax / 448.f : 1.f;
  const float rinv = amax > 0.f ? f * (448.f / amax) : 0.f;
  if (lane == 0) scales[(size_t)bh * ((N + 63) >> 6) + rt] = scale;

  // codes of this row into LDS (D bytes per row, 16-byte chunks swizzled by
  // the row), then written out 1 KB per wave instruction
  constexpr int CB = D;                 // code bytes per row
  constexpr int CCH = CB / 16;
  __syncthreads();                      // every row has been read from the tile
#pragma unroll
  for (int c = 0; c < CCH; ++c) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float t[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        t[u] = fminf(fmaxf(v[16 * c + 4 * e + u] * rinv, -448.f), 448.f);
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], pk, true);
      w[e] = (uint32_t)pk;
    }
    *reinterpret_cast<u32x4*>(tile + r * CB + 16 * (c ^ (r % CCH))) = u32x4{w[0], w[1], w[2], w[3]};
  }
  __syncthreads();
  uint8_t* out = codes + head + (size_t)r0 * D;
#pragma unroll
  for (int i = 0; i < ROWS * CB / 1024; ++i) {
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
    hipLaunchKernelGGL((fa_fp8_quant_kernel<D, true>), dim3((unsigned)grid), dim3(64), 0, st,
                       (const bf16*)a.x, a.signs, (uint8_t*)a.codes, a.scales, a.N, rtiles);
  else
    hipLaunchKernelGGL((fa_fp8_quant_kernel<D, false>), dim3((unsigned)grid), dim3(64), 0, st,
                       (const bf16*)a.x, a.signs, (uint8_t*)a.codes, a.scales, a.N, rtiles);
  return hipGetLastError();
}

hipError_t launch_fp8_quant(const QuantArgs& a) {
  return a.d == 128 ? launch_quant_d<128>(a) : launch_quant_d<64>(a);
}

}  // namespace fa
