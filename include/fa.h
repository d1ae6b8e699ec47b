/*
 * fa.h -- exact attention (FlashAttention forward and backward, split-KV
 * decode with per-head or grouped K/V heads) on
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * What is computed (per batch b, head h; row-major [B, H, N, d] tensors,
 * the (batch, heads, seq_len, head_dim) layout of the "Flash Attention"
 * Markdown note, section "问题分析" / problem analysis):
 *
 *     s_ij  = scale * <q_i, k_j>          (j > i masked when causal)
 *     O_i   = sum_j softmax_j(s_ij) * v_j
 *     LSE_i = ln sum_j exp(s_ij)          (natural log, fp32)
 *
 * The N x N score matrix is never written to memory: queries are tiled in
 * the outer loop and keys/values in the inner loop with a running row max
 * and running sum (same note, "Tiling（分块）技术" and "递归计算softmax";
 * the FlashAttention-2 overview's Q-outer / KV-inner loop order).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never frees or retains them.  They must be non-NULL and
 *     16-byte aligned; tensors are dense (contiguous) in the stated layout.
 *   - Calls are asynchronous on the given stream (NULL = the default
 *     stream); results are valid after the caller synchronises.
 *   - Argument errors are reported by the return value before anything is
 *     launched; nothing crosses the ABI as an exception.  A launch failure
 *     returns FA_ERR_HIP (fa_last_error() has the HIP text); faults inside a
 *     kernel surface at the caller's next synchronisation.
 *   - Calls that share a library-owned workspace (fa_decode_splitkv, and
 *     fa_decode_splitkv_gqa, fa_decode_splitkv_varlen, fa_bwd, fa_bwd_ex or
 *     fa_bwd_varlen with a NULL workspace) on one device must not run
 *     concurrently on different streams.  From several host threads on one stream they are
 *     safe: each call queues all of its launches while holding the
 *     workspace lock, so the buffer is neither freed nor shared between
 *     the launches of one call.  Growing that workspace synchronises the
 *     device (hipDeviceSynchronize), so such calls are not for graph
 *     capture; pass a workspace there.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size, bad scale */
  FA_ERR_UNSUPPORTED = 2,   /* valid request this build does not implement (e.g. d=96) */
  FA_ERR_WORKSPACE = 3,     /* workspace too small or could not be allocated */
  FA_ERR_HIP = 4            /* the HIP runtime reported an error */
} fa_status;

typedef enum {
  FA_BF16 = 0,
  FA_FP32 = 1,
  FA_FP8_E4M3 = 2,          /* OCP E4M3FN (bias 7, max 448), block-scaled */
  FA_FP16 = 3               /* IEEE binary16 */
} fa_dtype;

/*
 * fa_fwd -- attention forward pass, bf16 in, bf16 out, fp32 LSE.
 *
 * q, k, v : bf16 [B, H, N, d]      o : bf16 [B, H, N, d]
 * lse     : fp32 [B, H, N]         (natural-log log-sum-exp of the scaled scores)
 * d in {64, 128}; N >= 1 (any length; tails are masked); B, H >= 1;
 * one (b, h) slice of q/k/v must be under 4 GiB (N * d * 2 < 2^32), else
 * FA_ERR_UNSUPPORTED;
 * scale finite and > 0 (the usual value is 1/sqrt(d), the softmax_scale
 * default of the flash_attn_func call in the note's "框架集成" section);
 * causal != 0 masks key j > query i (the causal=True option of the note's
 * "使用注意事项" usage notes).  Runs on the default stream.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, float scale, int causal);

/*
 * fa_fwd_ex -- the forward pass with dtype and stream options.
 *
 * in_dtype  FA_BF16     : q, k, v bf16 [B,H,N,d]; q_scale/k_scale/v_scale must be NULL.
 * in_dtype  FA_FP8_E4M3 : q, k, v E4M3FN codes [B,H,N,d] (1 byte each) with
 *                         one fp32 scale per 64 consecutive rows of each
 *                         (b, h): q_scale, k_scale, v_scale fp32
 *                         [B, H, ceil(N/64)], finite and > 0; element
 *                         value = code * scale (the block quantisation of
 *                         the FlashAttention-3 snippets).  Both products run
 *                         on fp8 matrix cores with fp32 accumulation: the
 *                         unnormalised probabilities (at most 2^0.75 each)
 *                         are multiplied by 256 and rounded to E4M3FN for
 *                         the P*V product, and each V block's scale is
 *                         applied exactly outside that rounding; the row
 *                         sum uses the unrounded fp32 values.  Within one
 *                         (b, h), a V block scale more than 2^127 below
 *                         the largest has its binary exponent raised to
 *                         127 below the largest's.
 *                         d must be 128 and out_dtype FA_BF16 (else
 *                         FA_ERR_UNSUPPORTED).
 * in_dtype  FA_FP16     : q, k, v IEEE fp16 [B,H,N,d] (the note's "使用注意事项"
 *                         usage notes list FP16 beside BF16); the same
 *                         kernel on the fp16 matrix cores, with P rounded
 *                         to fp16 for the P*V product; d in {64, 128}; no
 *                         scales.
 * out_dtype FA_BF16 (bf16 inputs), FA_FP16 (fp16 inputs) or FA_FP32 (either):
 *                         o is [B,H,N,d] of that type; any other pairing is
 *                         FA_ERR_INVALID_ARG.
 * lse fp32 [B,H,N] (required).  stream is a hipStream_t (NULL = default).
 */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  int in_dtype;   /* fa_dtype */
  int out_dtype;  /* fa_dtype */
  int B, H, N, d;
  float scale;
  int causal;
  void* stream;
} fa_fwd_params;

fa_status fa_fwd_ex(const fa_fwd_params* p);

/*
 * fa_decode_splitkv -- single-query decode with the KV length split across
 * workgroups (the Flash-Decoding scheme of the FlashAttention-2 overview
 * snippets: K and V cut into parts, each part gives a partial output, the
 * partial outputs are merged; the FlashAttention-3 snippets call the merge
 * the splitK combine).
 *
 * q      : bf16 [B, H, 1, d]          o : bf16 [B, H, 1, d]
 * kcache, vcache : bf16 [B, H, Lkv, d]   (no mask; every key is visible)
 * num_splits in [1, Lkv]: split s covers keys [s*c, min((s+1)*c, Lkv)),
 * c = ceil(Lkv / num_splits).  scale = 1/sqrt(d).  d in {64, 128}.
 * One split must span under 4 GiB (c * d * 2 < 2^32), else FA_ERR_UNSUPPORTED.
 * Each split writes a normalised partial O_s and its LSE_s (fp32) to a
 * workspace; a second kernel merges them with weights exp(LSE_s - LSE).
 * The workspace is owned by the library, grown on demand per device and
 * kept until the process ends (it allocates; see fa_decode_splitkv_ex for
 * a caller-provided workspace).  Default stream.
 */
fa_status fa_decode_splitkv(const void* q, const void* kcache, const void* vcache, void* o,
                            int B, int H, int Lkv, int d, int num_splits);

/* Bytes of workspace fa_decode_splitkv_ex needs: B*H*num_splits*(d+1)*4,
 * rounded up to 256.  Returns 0 for arguments fa_decode_splitkv would reject. */
size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits);

/*
 * fa_decode_splitkv_ex -- as fa_decode_splitkv, plus: an explicit softmax
 * scale (finite, > 0); lse fp32 [B, H] (may be NULL); a caller-owned device
 * workspace of at least fa_decode_workspace_bytes() bytes (16-byte aligned;
 * FA_ERR_WORKSPACE if smaller); and a stream.  Layout of the workspace after
 * the call: partial O fp32 [B, H, num_splits, d], then partial LSE fp32
 * [B, H, num_splits] (an empty split has O = 0, LSE = -inf).
 */
fa_status fa_decode_splitkv_ex(const void* q, const void* kcache, const void* vcache, void* o,
                               float* lse, int B, int H, int Lkv, int d, int num_splits,
                               float scale, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * fa_decode_splitkv_noalloc -- fa_decode_splitkv_ex for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and arguments, with the
 * split partials kept in a fixed scratch array inside the library instead of
 * a workspace.  The call makes no hipMalloc/hipFree and no host allocation
 * on its success path.
 *
 * Limit: the partials, fa_decode_workspace_bytes(B, H, d, num_splits) =
 * B*H*num_splits*(d+1)*4 bytes rounded up to 256, must fit in
 * FA_DECODE_SCRATCH_BYTES (32 MiB; e.g. B=8, H=32, d=128 up to 254 splits),
 * else FA_ERR_WORKSPACE and nothing is launched.  Each GPU the library runs
 * on holds its own copy of the scratch until the process ends; the first
 * call on a device looks up its address there.  Every call on one GPU
 * shares that GPU's scratch, so calls that overlap on one GPU (concurrent
 * streams, several host threads without ordering) race and give wrong
 * results: serialise them, e.g. on one stream.  Nothing in the scratch
 * needs clearing: each call writes every partial it reads.
 * Other arguments, layouts and errors as fa_decode_splitkv_ex.
 */
#define FA_DECODE_SCRATCH_BYTES (32u << 20)
fa_status fa_decode_splitkv_noalloc(const void* q, const void* kcache, const void* vcache, void* o,
                                    float* lse, int B, int H, int Lkv, int d, int num_splits,
                                    float scale, void* stream);

/*
 * fa_decode_splitkv_gqa -- single-query split-KV decode where several query
 * heads share one key/value head (grouped-query attention; multi-query
 * attention when Hkv = 1: the MQA note among the related posts of the CSDN
 * "flash attention CUDA programming, pipeline-parallel acceleration V6"
 * page, where keys and values keep a single shared head and queries keep
 * all of theirs).  Query head h attends over key/value head h / (Hq / Hkv).
 *
 * q      : bf16 [B, Hq, 1, d]          o   : bf16 [B, Hq, 1, d]
 * kcache, vcache : bf16 [B, Hkv, Lkv, d]   lse : fp32 [B, Hq] or NULL
 * Hkv >= 1 must divide Hq (else FA_ERR_INVALID_ARG); Hkv = Hq is plain
 * multi-head decode.  num_splits, d, scale and the 4 GiB-per-split limit
 * are as for fa_decode_splitkv_ex, and so is the workspace: at least
 * fa_decode_workspace_bytes(B, Hq, d, num_splits) bytes holding partial O
 * fp32 [B, Hq, num_splits, d] then partial LSE fp32 [B, Hq, num_splits]
 * after the call.  workspace = NULL with workspace_bytes = 0 selects the
 * library-owned workspace (which allocates, see fa_decode_splitkv).
 * One workgroup streams a (batch, K/V head, split) range once for up to 16
 * query heads of its group (G = Hq / Hkv <= 16) or up to 32 (G > 16);
 * groups larger than 32 read the range once per 32 heads.
 */
fa_status fa_decode_splitkv_gqa(const void* q, const void* kcache, const void* vcache, void* o,
                                float* lse, int B, int Hq, int Hkv, int Lkv, int d,
                                int num_splits, float scale, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * fa_decode_splitkv_varlen -- fa_decode_splitkv_gqa over a padded cache with
 * a length per sequence (a serving batch whose sequences have different
 * numbers of cached tokens): sequence b attends over the first
 * Lb = seqlens_k[b] keys of its cache (clamped to [0, Lkv]).  Its keys are
 * cut into num_splits ranges of c_b = ceil(Lb / num_splits): split s covers
 * [s*c_b, min((s+1)*c_b, Lb)).  A sequence with Lb = 0 gets O = 0 and
 * LSE = -inf.
 *
 * seqlens_k : int32 DEVICE array [B]; kcache, vcache : bf16 [B, Hkv, Lkv, d]
 * (Lkv the capacity).  Everything else as fa_decode_splitkv_gqa.
 */
fa_status fa_decode_splitkv_varlen(const void* q, const void* kcache, const void* vcache, void* o,
                                   float* lse, const int* seqlens_k, int B, int Hq, int Hkv,
                                   int Lkv, int d, int num_splits, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * fa_fwd_varlen -- the bf16 forward pass over a batch of packed sequences of
 * unequal lengths (the power-of-two length rule of the Flash Attention
 * note, "使用注意事项", does not apply: any lengths work).  Sequence b has
 * Lq = cu_seqlens_q[b+1] - cu_seqlens_q[b] queries and Lk =
 * cu_seqlens_k[b+1] - cu_seqlens_k[b] keys; Lq and Lk may differ.
 *
 * q, o   : bf16 [total_q, H, d] (token-major; sequence b at rows cu_seqlens_q[b]..)
 * k, v   : bf16 [total_k, H, d]
 * lse    : fp32 [H, total_q]
 * cu_seqlens_q, cu_seqlens_k : int32 DEVICE arrays of B+1 non-decreasing
 *          offsets starting at 0, ending at total_q / total_k.
 * max_seqlen_q, max_seqlen_k : bounds on Lq and Lk (they size the launch;
 *          longer sequences are cut to them).  The kernel clamps every
 *          offset to [0, total], so malformed offsets give wrong values but
 *          no access outside the tensors.
 * causal : masking aligned at the end of each sequence -- query i sees key
 *          j iff j <= i + (Lk - Lq): the queries are the last Lq positions
 *          of a length-Lk sequence, as for a prefill chunk against cached
 *          keys.  A query that sees no key (Lq > Lk) gets O = 0, LSE = -inf.
 * d in {64, 128}; bf16 output; one sequence's rows of one tensor must span
 * under 4 GiB (max_seqlen * H * d * 2 < 2^32), else FA_ERR_UNSUPPORTED.
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                        int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int d,
                        float scale, int causal, void* stream);

/*
 * fa_fp8_quantize -- bf16 -> the fp8 forward pass's input format, with the
 * optional incoherent processing of the FlashAttention-3 snippets (named
 * there beside block quantisation as the way FA-3 lowers fp8 error; read
 * here as a random orthogonal rotation of the head dimension).
 *
 * x      : bf16 [B, H, N, d]              codes  : uint8 E4M3FN [B, H, N, d]
 * signs  : fp32 [d] of +1/-1, or NULL     scales : fp32 [B, H, ceil(N/64)]
 * With signs, every row is first replaced by x diag(signs) H_d / sqrt(d)
 * (H_d the Sylvester-ordered Walsh-Hadamard matrix).  Quantise Q and K with
 * the same signs (Q K^T is unchanged) and V with NULL.  Then, per 64-row
 * block, scale = max|x| / 448 (1 for an all-zero block) and each code is
 * the fp32 ratio x * (448 / max|x|) -- within about an ulp of x / scale --
 * rounded to nearest, ties to even (so a value within an ulp of a rounding
 * midpoint of x / scale may take either neighbour).  d in {64, 128}, else
 * FA_ERR_UNSUPPORTED.  x and codes 16-byte aligned.
 */
fa_status fa_fp8_quantize(const void* x, const float* signs, void* codes, float* scales, int B,
                          int H, int N, int d, void* stream);

/*
 * fa_fp8_quantize_ex -- fa_fp8_quantize with a choice of the block scale.
 * FA_FP8_SCALE_AMAX is fa_fp8_quantize's max|x| / 448.  FA_FP8_SCALE_POW2
 * takes the smallest power of two with max|x| / scale <= 448 (1 for an
 * all-zero block): the E8M0 form of the matrix cores' operand scale.  For
 * V this is the fast form: the fp8 forward pass applies a power of two to
 * V's products inside the MFMA, and when all of a head's V scales share one
 * mantissa it needs no per-block multiply of its accumulator.  Q and K are
 * better kept at max|x| / 448, which makes each block's largest element
 * exact (their scales cost nothing in the forward pass).  With the POW2 rule
 * and no rotation, x / scale is exact and the codes are the nearest-even
 * E4M3FN values of it.  Other scale_rule values: FA_ERR_INVALID_ARG.  The
 * rest as fa_fp8_quantize.
 */
typedef enum {
  FA_FP8_SCALE_AMAX = 0,
  FA_FP8_SCALE_POW2 = 1
} fa_fp8_scale_rule;

fa_status fa_fp8_quantize_ex(const void* x, const float* signs, void* codes, float* scales,
                             int B, int H, int N, int d, int scale_rule, void* stream);

/*
 * fa_bwd -- gradients of exact attention: dQ, dK, dV for an upstream dO,
 * with P recomputed from Q, K and the forward pass's LSE (the recomputation
 * of the FlashAttention summaries; the FlashAttention-2 overview, section
 * 3.4, on splitting the backward pass over thread blocks; the Flash
 * Attention note, "使用注意事项", on fp32 softmax statistics in the backward
 * pass).  With s_ij = scale * <q_i, k_j> (j > i masked when causal),
 * P = exp(s - LSE), D_i = sum_c dO_ic * O_ic:
 *     dV = P^T dO,   dS = P * (dO V^T - D),   dQ = scale * dS K,
 *     dK = scale * dS^T Q.
 *
 * q, k, v, o, dout, dq, dk, dv : bf16 [B, H, N, d]   lse : fp32 [B, H, N]
 * o and lse are the forward pass's outputs for the same q, k, v, scale and
 * causal flag (fa_fwd / fa_fwd_ex with bf16 output).  d in {64, 128}, else
 * FA_ERR_UNSUPPORTED; scale finite and > 0.  All pointers 16-byte aligned.
 * The workspace holds -D and -LSE/scale (two fp32 [B, H, N] arrays): at
 * least fa_bwd_workspace_bytes(B, H, N) bytes, or NULL with workspace_bytes
 * = 0 to use the library-owned workspace (which allocates).  dq, dk and dv are
 * written in full (no accumulation into existing contents); the result is
 * deterministic (no atomics).
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N);

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                 float scale, int causal, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * fa_bwd_ex -- fa_bwd with the tensor type as an argument: dtype FA_BF16
 * (exactly fa_bwd) or FA_FP16, for the mixed-precision training of the Flash
 * Attention note's "使用注意事项" usage notes (an fp16 forward pass, fp32
 * softmax statistics in the backward pass).  With FA_FP16, q, k, v, o, dout,
 * dq, dk and dv are IEEE fp16 [B, H, N, d] (o and lse from fa_fwd_ex with
 * in_dtype = out_dtype = FA_FP16); P and dS are rounded to fp16 for the
 * matrix cores, D and the accumulation stay fp32.  Any other dtype is
 * FA_ERR_INVALID_ARG.  Everything else is as for fa_bwd.
 */
fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                    float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * fa_bwd_varlen -- fa_bwd over a batch of packed sequences of unequal
 * lengths: the gradients of fa_fwd_varlen's output (the Flash Attention
 * note's "使用注意事项" lifts the power-of-two length rule; the backward
 * pass is the same recomputation as fa_bwd, per sequence).  Sequence b has
 * Lq = cu_seqlens_q[b+1] - cu_seqlens_q[b] queries and Lk =
 * cu_seqlens_k[b+1] - cu_seqlens_k[b] keys.
 *
 * q, o, dout, dq : bf16 [total_q, H, d]     k, v, dk, dv : bf16 [total_k, H, d]
 * lse            : fp32 [H, total_q], fa_fwd_varlen's output for the same
 *                  q, k, v, offsets, scale and causal flag (o likewise).
 * cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal : as for
 *          fa_fwd_varlen (masking aligned at the end of each sequence).  A
 *          query that sees no key gets dQ = 0; keys of a sequence without
 *          queries get dK = dV = 0.  Rows outside every sequence's range are
 *          not written.
 * The workspace holds -D and -LSE/scale (two fp32 [H, total_q] arrays): at
 * least fa_bwd_workspace_bytes(1, H, total_q) bytes, or NULL with
 * workspace_bytes = 0 for the library-owned workspace (which allocates).
 * d in {64, 128}, else FA_ERR_UNSUPPORTED; scale finite and > 0; pointers to
 * tensors 16-byte aligned, offsets 4-byte aligned.  One sequence's rows of
 * one tensor must span under 4 GiB (max_seqlen * H * d * 2 < 2^32), else
 * FA_ERR_UNSUPPORTED.  Deterministic (no atomics).
 */
fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                        int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int d,
                        float scale, int causal, void* workspace, size_t workspace_bytes,
                        void* stream);

/* A static string naming the status. */
const char* fa_status_string(fa_status s);

/* The message of the last failing call on this thread ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
