// Launcher interface between the C-ABI host layer (fa_api.cpp) and the HIP
// kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* q_scale;  // fp8 only
  const float* k_scale;
  const float* v_scale;
  int B, H, N, d;
  float scale;        // softmax scale
  float scale_log2;   // scale * log2(e)
  int causal;
  // packed sequences of unequal lengths (bf16 path): q, k, v, o are
  // [total, H, d] token-major, lse is [H, total_q]; sequence b occupies rows
  // cu_q[b]..cu_q[b+1] (queries) and cu_k[b]..cu_k[b+1] (keys).  N is the
  // largest query length, Nk the largest key length.  Null cu_q: dense
  // [B, H, N, d] tensors with as many keys as queries.
  const int* cu_q;
  const int* cu_k;
  int Nk, total_q, total_k;
  int out_f32;
  int in_f16;         // q, k, v (and a 16-bit o) are IEEE fp16 instead of bf16
  void* stream;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;         // may be null
  float* part_o;      // [B*H, S, d] fp32
  float* part_lse;    // [B*H, S]    fp32
  int B, H, Lkv, d, num_splits;
  int Hkv;            // key/value heads (H for plain multi-head decode)
  const int* seqlens_k;  // [B] keys per sequence in the padded cache, or null (all Lkv)
  float scale_log2;
  void* stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;   // [B*H, N] natural log, from the forward pass
  float* ndsum;       // [B*H, N] workspace: -rowsum(dO * O)
  float* nlse;        // [B*H, N] workspace: -LSE / scale
  void* dq;
  void* dk;
  void* dv;
  int B, H, N, d;
  float scale;
  float scale_log2;
  int causal;
  int in_f16;         // fp16 tensors instead of bf16
  // packed sequences of unequal lengths (bf16): q, o, dout, dq are
  // [total_q, H, d], k, v, dk, dv [total_k, H, d], lse, ndsum and nlse
  // [H, total_q];
  // sequence b at rows cu_q[b].. and cu_k[b]..  N and Nk bound the query and
  // key lengths.  Null cu_q: the dense [B, H, N, d] layout.
  const int* cu_q;
  const int* cu_k;
  int Nk, total_q, total_k;
  void* stream;
};

struct QuantArgs {
  const void* x;        // bf16 [B, H, N, d]
  const float* signs;   // [d] +-1, or null for no rotation
  void* codes;          // u8 [B, H, N, d]
  float* scales;        // [B, H, ceil(N/64)]
  int B, H, N, d;
  int pow2;             // power-of-two scales (else max|x| / 448)
  void* stream;
};

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fp8_quant(const QuantArgs& a);
hipError_t launch_bwd(const BwdArgs& a);
hipError_t launch_fwd_fp8(const FwdArgs& a);
hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_decode_gqa(const DecodeArgs& a);
// the merge of the split partials (shared by both decode paths)
hipError_t launch_decode_combine(const DecodeArgs& a);

// The library's fixed decode scratch (for the entry point that allocates
// nothing): its device address on the current device, looked up once per
// device.  kDecodeScratchBytes is FA_DECODE_SCRATCH_BYTES of fa.h.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace fa
