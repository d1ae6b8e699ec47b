// Device-side helpers shared by the gfx950 attention kernels: vector types,
// MFMA wrappers, wave64 cross-lane reductions and bf16 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t as_u32(float x) { return __builtin_bit_cast(uint32_t, x); }

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16) on the matrix cores.
// Operand layout (wave64): lane l supplies row (A) / column (B) l%32 and
// eight consecutive contraction slots 8*(l/32)..+7.  Result layout: lane l
// holds column l%32, rows 8*(i/4) + 4*(l/32) + i%4 for i = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same product on IEEE fp16 operands: the eight halves of a lane travel
// in the same 16 bytes (bf16x8 is used as the carrier of 16-bit bits).
__device__ __forceinline__ f32x16 mfma32x32x16_f16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies row
// (A) / column (B) l%16 and contraction slots 8*(l/16)..+7; the result lane l
// holds column l%16, rows 4*(l/16) + i for i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Rows of 16 lanes exchange a value with the neighbouring row: returns
// {x[l], x[l^16]} in some order.
__device__ __forceinline__ float max_pair16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  return fmaxf(as_f32(r[0]), as_f32(r[1]));
}
__device__ __forceinline__ float sum_pair16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  return as_f32(r[0]) + as_f32(r[1]);
}

// Both halves of the wave exchange a value: returns {x[l%32], x[32 + l%32]}
// in some order, so op(r.x, r.y) is the pairwise reduction over l and l^32.
__device__ __forceinline__ float max_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  return fmaxf(as_f32(r[0]), as_f32(r[1]));
}
__device__ __forceinline__ float sum_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  return as_f32(r[0]) + as_f32(r[1]);
}

// DPP lane permutations within 16-lane rows.
enum : int {
  kDppQuadXor1 = 0xB1,        // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,        // quad_perm [2,3,0,1]
  kDppRowMirror = 0x140,      // lane i <- lane 15-i (within 16)
  kDppRowHalfMirror = 0x141,  // lane i <- lane 7-i (within 8)
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return as_f32(__builtin_amdgcn_mov_dpp(as_u32(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G = 8 or 16); every lane gets the total.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(G == 8 || G == 16, "group of 8 or 16 lanes");
  if constexpr (G == 16) x += dpp<kDppRowMirror>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppQuadXor1>(x);
  return x;
}

// v_dot2_f32_bf16: acc + a.lo*b.lo + a.hi*b.hi for bf16 pairs packed in dwords.
// (The operands are plain dwords: a bit_cast applied to a vector element
// expression directly has been seen to read element 0 only.)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         acc, false);
}

// bf16 pair (packed in a dword) -> two floats.
__device__ __forceinline__ float bf16lo(uint32_t w) { return as_f32(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return as_f32(w & 0xFFFF0000u); }

// The same for fp16 pairs.
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
}
__device__ __forceinline__ float f16lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[0]; }
__device__ __forceinline__ float f16hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[1]; }

// Buffer resource over [base, base + bytes): loads past the end return 0,
// which is how the kernels read tiles that overhang the sequence without a
// branch.  Offsets are 32-bit byte offsets from base.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// The same with the non-temporal hint (for data read exactly once).
__device__ __forceinline__ u32x4 buf_load16_nt(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

__device__ __forceinline__ u32x2 buf_load8_nt(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2));
}

// Direct global->LDS copies (buffer_load ... lds) of 16 or 4 bytes per lane
// to lds + 16 * lane (or + 4 * lane).  Issued through inline asm rather than
// the LDS-DMA builtin: after the builtin the compiler puts a vmcnt(0) wait in
// front of the next transposing LDS read (ds_read_b64_tr_b16), whatever LDS
// it reads, which makes a tile prefetch complete before the first transposed
// product of the tile it is meant to overlap.  The copies write no registers;
// the kernel itself waits for them (vmcnt(0), then a barrier) before any wave
// reads the stage they fill.  M0 carries the LDS address.
__device__ __forceinline__ void lds_dma16(rsrc_t r, const void* lds, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t la = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds;
  asm volatile("buffer_load_dwordx4 %1, %2, 0 offen lds" ::"{m0}"(la), "v"(off), "s"(r) : "memory");
#endif
}
__device__ __forceinline__ void lds_dma4(rsrc_t r, const void* lds, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t la = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds;
  asm volatile("buffer_load_dword %1, %2, 0 offen lds" ::"{m0}"(la), "v"(off), "s"(r) : "memory");
#endif
}

// Round two floats to bf16 (nearest even) and pack them (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 p = {(bf16)a, (bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// Round two floats to fp16 (nearest even) and pack them (a in the low half).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2 p = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// The 16-bit element type of a forward pass: bf16, or fp16 when F16.
template <bool F16>
__device__ __forceinline__ f32x16 mma16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  if constexpr (F16) return mfma32x32x16_f16(a, b, c);
  else return mfma32x32x16(a, b, c);
}
template <bool F16>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  if constexpr (F16) return pack_f16(a, b);
  else return pack_bf16(a, b);
}
template <bool F16>
__device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (F16) return f16lo(w);
  else return bf16lo(w);
}
template <bool F16>
__device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (F16) return f16hi(w);
  else return bf16hi(w);
}
template <bool F16>
__device__ __forceinline__ float dot2_16(uint32_t a, uint32_t b, float acc) {
  if constexpr (F16) return dot2_f16(a, b, acc);
  else return dot2_bf16(a, b, acc);
}

// Store a wave's 32 x D tile of 16-bit outputs held in the 32x32 MFMA
// accumulator layout (lane l: row l%32; acc[cb][i] is feature
// 32cb + 8(i/4) + 4(l/32) + i%4), each value times mul, as whole rows: the
// tile is staged in LDS (32 * 2D bytes at lds, 16-byte chunks XOR-swizzled
// by row so that both passes are free of bank conflicts) and read back so
// that 2D/16 lanes store one row, instead of 8 bytes per row and lane.
// row(r) is the destination of tile row r; rows r >= nrows are not written.
// The caller guarantees that nothing else uses those LDS bytes meanwhile.
template <bool F16, int D, typename RowPtr>
__device__ __forceinline__ void store_tile_rows(uint8_t* lds, const f32x16 (&acc)[D / 32], float mul,
                                                int lane, int nrows, RowPtr row) {
  constexpr int RB = D * 2, NCH = RB / 16;
  const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int ch = 4 * cb + ii;
      *reinterpret_cast<u32x2*>(lds + l32 * RB + 16 * (ch ^ (l32 % NCH)) + 8 * g) =
          u32x2{pack16<F16>(acc[cb][4 * ii] * mul, acc[cb][4 * ii + 1] * mul),
                pack16<F16>(acc[cb][4 * ii + 2] * mul, acc[cb][4 * ii + 3] * mul)};
    }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave's rows are in LDS
#pragma unroll
  for (int k = 0; k < 32 * NCH / 64; ++k) {
    const int L = 64 * k + lane, r = L / NCH, ch = L % NCH;
    const u32x4 val = *reinterpret_cast<const u32x4*>(lds + r * RB + 16 * (ch ^ (r % NCH)));
    if (r < nrows) *reinterpret_cast<u32x4*>(row(r) + 8 * ch) = val;
  }
}

}  // namespace fa
