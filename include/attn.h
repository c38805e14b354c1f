/*
 * attn.h -- C ABI of the MI355X (gfx950) fused attention forward.
 *
 * The library computes, for every batch b, head h and query i,
 *
 *     O[b,h,i,:] = softmax_j( scale * Q[b,h,i,:] . K[b,h,j,:]
 *                             + bias[b,h,i/64,j/64] ) V[b,h,j,:]
 *
 * over the keys j the mask allows (causal: j <= i).  This is the attention
 * formula of page 4 ("FlashAttention (TR)", section on the problems of
 * standard attention), with the masking step of the single fused kernel
 * (same page, section on fusing all operations into one kernel) and the
 * optional additive log-form gate of page 5 ("SAS", the log-form gate placed
 * inside the attention softmax).  The N x N score matrix never reaches
 * device memory: keys are processed in blocks with a running maximum and a
 * running sum (page 4, online softmax section) inside one kernel that
 * writes only the final output (page 4, fused kernel section).
 *
 * The 8-bit path follows page 1 ("SageAttention", claim vs reality
 * section): K is mean-centred over tokens, Q K^T runs in INT8 with one fp32
 * scale per 64-row block, P goes to FP8 e4m3 for the P V product, and the
 * products are accumulated in two levels in fp32.
 *
 * Conventions for every entry point:
 *  - Tensors are contiguous [B,H,N,d], d innermost, in device memory, with
 *    16-byte aligned base pointers.  d must be 64, 96 or 128; B, H, N >= 1;
 *    B*H*N*d must fit in 2^31 elements per tensor.
 *  - The caller owns every buffer.  The library allocates no device memory,
 *    keeps no mutable state between calls and is safe to call from several
 *    host threads (on distinct output buffers).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *    stream) and may be recorded into a HIP graph: they launch kernels only
 *    (no allocation, no memset, no host synchronisation).  Every argument
 *    check runs before any launch: a non-zero status means nothing was
 *    launched and nothing was written.  Faults of the device itself surface
 *    at stream synchronisation.
 *  - There is no fallback path: an unsupported shape, dtype or device is an
 *    error, never a slower materialising implementation (page 3, the
 *    glossary entry's warning about silent fallbacks).
 *  - NaN or Inf in the inputs propagate.  A row whose every key is masked
 *    (possible only through -inf bias entries) gives O = 0 and LSE = -inf.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 9

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,      /* a required pointer is NULL                   */
    ATTN_ERR_SHAPE = 2,     /* B, H or N < 1, or a tensor exceeds 2^31 elts */
    ATTN_ERR_HEADDIM = 3,   /* d is not 64, 96 or 128                       */
    ATTN_ERR_DTYPE = 4,     /* unsupported input/output dtype combination   */
    ATTN_ERR_ALIGN = 5,     /* a pointer is not 16-byte aligned             */
    ATTN_ERR_ARG = 6,       /* scale not finite, causal not 0/1, ...        */
    ATTN_ERR_WORKSPACE = 7, /* workspace NULL or smaller than required      */
    ATTN_ERR_DEVICE = 8,    /* current device is not gfx950                 */
    ATTN_ERR_HIP = 9        /* a HIP runtime call or a launch failed        */
} attn_status;

/* Element types of inputs and outputs. */
typedef enum {
    ATTN_DTYPE_F16 = 0,
    ATTN_DTYPE_BF16 = 1,
    ATTN_DTYPE_F32 = 2
} attn_dtype;

/* Number format of Q and K in the 8-bit path's workspace. */
typedef enum {
    ATTN_QK_INT8 = 0,      /* the INT8 recipe (attn_k_smooth_quant)            */
    ATTN_QK_FP8 = 1,       /* the FP8-QK variant (attn_k_smooth_quant_fp8qk)   */
    ATTN_QK_INT8_NO_V = 2  /* INT8 Q and K only, for attn_fwd_sage8_pv16: V
                              is not read and the workspace's V regions are
                              not written (preparation only)                  */
} attn_qk_format;

/*
 * attn_fwd_f16 / attn_fwd_bf16 -- fused attention forward (fp16 / bf16).
 *
 *  q, k, v    [B,H,N,d] fp16 (attn_fwd_f16) or bf16 (attn_fwd_bf16), read only.
 *  o          [B,H,N,d] output; out_dtype is the input dtype or ATTN_DTYPE_F32.
 *  lse        [B,H,N] fp32 natural-log log-sum-exp of each row's scaled,
 *             biased scores (nullable: not written when NULL).
 *  causal     0 or 1; 1 lets query i see keys j <= i.
 *  scale      finite multiplier of Q.K (1/sqrt(d) for standard attention).
 *  bias       nullable fp32 [B,H,nb,nb], nb = ceil(N/64): additive logit
 *             (natural-log units, not multiplied by scale) for each
 *             64-query x 64-key block.  -inf entries mask whole blocks.
 *             With a bias, B*H*nb*nb must be below 2^31 and nb below 32768
 *             (N <= 2,097,088), else ATTN_ERR_SHAPE.
 *  Products run on the matrix cores with fp32 accumulation; P is rounded
 *  to the input dtype for the P V product.
 */
attn_status attn_fwd_f16(const void* q, const void* k, const void* v, void* o,
                         float* lse, int B, int H, int N, int d, int causal,
                         float scale, const float* bias, int out_dtype,
                         void* stream);
attn_status attn_fwd_bf16(const void* q, const void* k, const void* v, void* o,
                          float* lse, int B, int H, int N, int d, int causal,
                          float scale, const float* bias, int out_dtype,
                          void* stream);

/*
 * attn_fwd_strided_f16 / attn_fwd_strided_bf16 -- the same forward on
 * tensors of any layout with d contiguous, and on packed sequences of
 * different lengths (the drop-in layouts of the SageAttention page's
 * integration section and of a scaled-dot-product-attention call: e.g.
 * [B,N,H,d] token-major tensors, or q/k/v as views of one fused projection).
 *
 *  strides    host array of 12 element strides: for q, k, v, o in turn the
 *             (batch, head, token) strides; d is contiguous.  Each stride is
 *             >= 0 and a multiple of 8 elements (16-byte rows), each token
 *             stride >= d, and (N + 64) * token stride * 2 < 2^32 bytes
 *             (the last key block reads whole 64-row blocks; rows past N
 *             read as zeros).
 *  cu_seqlens nullable device int32 [B+1]: packed sequences.  Sequence b is
 *             tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of the token axis
 *             (the batch strides are then unused) and attends only within
 *             itself; N is the longest length.  The values are read on the
 *             device and not validated: they must be non-decreasing with
 *             every length <= N (longer lengths are clamped to N).
 *  lse        nullable fp32 [B,H,N] (row b,h,i for i < the sequence length).
 *  bias       nullable fp32 [B,H,nb,nb] contiguous, nb = ceil(N/64): the
 *             block bias of attn_fwd_f16 / attn_fwd_bf16 (page 5, "SAS",
 *             log-form gate).  With cu_seqlens, sequence b takes
 *             bias[b,h,i,j] for its query block i and key block j, both
 *             counted from its own first token (N, and so nb, from the
 *             longest length).
 *  Other arguments as attn_fwd_f16 / attn_fwd_bf16.  The arithmetic is that
 *  of attn_fwd_f16/bf16.  (ABI version 9 added the bias argument.)
 */
attn_status attn_fwd_strided_f16(const void* q, const void* k, const void* v, void* o,
                                 float* lse, int B, int H, int N, int d,
                                 const long long* strides, const int* cu_seqlens,
                                 int causal, float scale, const float* bias, int out_dtype,
                                 void* stream);
attn_status attn_fwd_strided_bf16(const void* q, const void* k, const void* v, void* o,
                                  float* lse, int B, int H, int N, int d,
                                  const long long* strides, const int* cu_seqlens,
                                  int causal, float scale, const float* bias, int out_dtype,
                                  void* stream);

/*
 * attn_sage8_workspace_size -- bytes of device workspace that
 * attn_k_smooth_quant fills and attn_fwd_sage8 reads for this shape
 * (0 when the shape is invalid).  The workspace holds the INT8 Q and K,
 * the FP8 V (in the layout the P V product reads), their fp32 scales and
 * the K mean; its layout is private to the library.
 */
size_t attn_sage8_workspace_size(int B, int H, int N, int d);

/*
 * attn_sage8_workspace_layout -- where the prepared data sit inside the
 * workspace, for inspection and tests.  Writes up to n values to out, in
 * this order: byte offsets of Qq, Kq, Vq, sQ, sK, sV, kmean, then the padded
 * token count Np and the number of 64-row blocks nblk.  Layouts: Qq, Kq int8
 * [B,H,Np,d]; sQ, sK fp32 [B,H,nblk]; sV, kmean fp32 [B,H,d]; Vq e4m3
 * [B,H,nblk,d,64] where byte 32h + 16T + 4g + u of a row holds key
 * 32T + 8g + 4h + u of the block (the operand order of the P V product).
 * Returns the number of values written, 0 for an invalid shape.
 */
int attn_sage8_workspace_layout(int B, int H, int N, int d, size_t* out, int n);

/*
 * attn_k_smooth_quant -- the 8-bit preparation (page 1, "SageAttention":
 * mean-centring of K before INT8 quantisation; FP8 for the second product).
 *
 *  q, k, v    [B,H,N,d] in in_dtype (ATTN_DTYPE_F16 or ATTN_DTYPE_BF16).
 *  workspace  device buffer of at least attn_sage8_workspace_size bytes,
 *             256-byte aligned; fully overwritten.
 *  Steps: kmean[b,h,c] = mean over all N tokens of K (sum in fp64, rounded
 *  once to fp32); INT8 codes of Q and of K - kmean with one scale per
 *  64-row block (scale = amax/127, code = rne(x * (127/amax)), clamped to
 *  +-127); e4m3 codes of V with one scale per (b,h,channel) (scale =
 *  amax/448, code = e4m3_rne(v * (448/amax))).  A zero amax gives scale 1.
 */
attn_status attn_k_smooth_quant(const void* q, const void* k, const void* v,
                                int in_dtype, int B, int H, int N, int d,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * attn_fwd_sage8 -- 8-bit fused forward from a prepared workspace.
 *
 *  workspace  written by attn_k_smooth_quant with the same B, H, N, d
 *             (the library cannot check this; the Python binding bundles
 *             the two so they cannot disagree).
 *  o          [B,H,N,d] in out_dtype (F16, BF16 or F32).
 *  lse, causal, scale, bias as for attn_fwd_bf16.
 *  S = Qq Kq^T in INT8 with int32 accumulation, dequantised with the two
 *  block scales; online softmax in fp32 with a running maximum m that is
 *  raised only when a 64-key block's maximum exceeds it by more than 2 (log2
 *  units); P^ = e4m3(448 * 2^(t - m - 2)) <= 448; each key block's P^ V
 *  partial accumulates in fp32 inside one matrix instruction (level 1) and
 *  is added to the rescaled running output in fp32 (level 2); the V scales
 *  and 1/l are applied once at the end.
 */
attn_status attn_fwd_sage8(const void* workspace, void* o, float* lse, int B,
                           int H, int N, int d, int causal, float scale,
                           const float* bias, int out_dtype, void* stream);

/*
 * attn_k_smooth_quant_fp8qk / attn_fwd_sage8_fp8qk -- the FP8-QK variant of
 * the 8-bit path: Q and the mean-centred K go to FP8 e4m3 with one scale
 * per 64-row block (scale = amax/448, code = e4m3_rne(x * (448/amax)); a
 * zero amax gives scale 1), the block-wise dynamic scaling that page 2
 * ("FlashAttention-3" bulletin, claim vs reality section) says FP8 products
 * need, and S = Q K^T runs on the FP8 matrix instruction in fp32.  K mean,
 * V, P and the two-level P V product are as in attn_k_smooth_quant /
 * attn_fwd_sage8, so the pair differs from the INT8 recipe only in the
 * number format of the first product.  The workspace (same size and
 * layout; Qq and Kq hold e4m3 bytes) must be written by
 * attn_k_smooth_quant_fp8qk for attn_fwd_sage8_fp8qk and by
 * attn_k_smooth_quant for attn_fwd_sage8; the library cannot tell them
 * apart.  At d = 96 the last 64-deep product covers channels 64..95 with
 * zero codes for the rest.  Other arguments as for the INT8 pair.
 */
attn_status attn_k_smooth_quant_fp8qk(const void* q, const void* k, const void* v,
                                      int in_dtype, int B, int H, int N, int d,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);
attn_status attn_fwd_sage8_fp8qk(const void* workspace, void* o, float* lse, int B,
                                 int H, int N, int d, int causal, float scale,
                                 const float* bias, int out_dtype, void* stream);

/*
 * attn_fwd_sage8_pv16 -- the 8-bit forward with INT8 scores and the 16-bit
 * P V product: the first product of page 1 ("SageAttention", claim vs
 * reality section: Q K^T in INT8 after K is mean-centred), while P and V
 * stay in the inputs' 16-bit format for the second product, as in
 * attn_fwd_bf16.  On the workloads measured this meets cos >= 0.999 and
 * rel-L1 <= 2e-2 against exact attention, which the FP8 P and V of
 * attn_fwd_sage8 do not (their rounding alone costs about 2-4% rel-L1).
 *
 *  workspace  written by attn_k_smooth_quant (INT8 format), or by
 *             attn_k_smooth_quant_strided with ATTN_QK_INT8_NO_V (no V
 *             statistics or codes: less preparation work), for the same B,
 *             H, N, d; only its Qq, Kq, scales and K mean are read.
 *  v          the 16-bit V [B,H,N,d] contiguous that was prepared, in
 *             v_dtype (ATTN_DTYPE_F16 or ATTN_DTYPE_BF16).
 *  o          [B,H,N,d] in out_dtype: v_dtype or ATTN_DTYPE_F32.
 *  lse, causal, scale, bias as for attn_fwd_bf16 (the LSE refers to the
 *  scores before the centring of K).
 *  S = Qq Kq^T in INT8 with int32 accumulation, dequantised with the two
 *  block scales; online softmax in fp32 as in attn_fwd_bf16 (running
 *  maximum raised lazily, P rounded to v_dtype for the product, fp32
 *  accumulation, one output write).  ABI version 8.
 */
attn_status attn_fwd_sage8_pv16(const void* workspace, const void* v, int v_dtype, void* o,
                                float* lse, int B, int H, int N, int d, int causal,
                                float scale, const float* bias, int out_dtype, void* stream);

/*
 * attn_k_smooth_quant_strided / attn_fwd_sage8_strided -- the 8-bit pair on
 * inputs and outputs of any layout with d contiguous (token-major [B,N,H,d],
 * views into a fused QKV projection, ...), so the 8-bit path takes the same
 * tensors as the 16-bit strided forward.  The computation and the workspace
 * are exactly those of the contiguous pair for the same logical [B,H,N,d]
 * data; qk_format (ATTN_QK_INT8 or ATTN_QK_FP8) selects the recipe (INT8, or
 * the FP8-QK variant) and must match between the two.
 *
 *  strides    host array of 9 element strides: (batch, head, token) of q,
 *             then k, then v.  Each a multiple of 8 and >= 0, token strides
 *             >= d, and (N + 256) * token stride * 2 < 2^32 (the column
 *             statistics read whole 256-token chunks; rows past N read as 0).
 *  o_strides  host array of 3 element strides (batch, head, token) of o,
 *             with the same rules (without the 256-token margin).
 *  cu_seqlens nullable device int32 [B+1]: packed sequences, as for
 *             attn_fwd_strided_f16.  Sequence b is tokens cu_seqlens[b] ..
 *             cu_seqlens[b+1]-1 of the token axis of q, k, v and o (the
 *             batch strides are then unused) and N is the longest length.
 *             The preparation treats each sequence as a batch entry of its
 *             own: K mean, V channel scales and the 64-row Q/K blocks are
 *             taken over that sequence alone, so its workspace slot and its
 *             rows of O are bit for bit those of a separate call on it.  The
 *             values are read on the device and not validated (non-decreasing,
 *             lengths <= N; longer lengths are clamped to N); a length of 0 is
 *             allowed.  Both calls must get the same array.  A bias is read
 *             as for attn_fwd_strided_f16: sequence b takes bias[b,h,i,j]
 *             for its query block i and key block j counted from its first
 *             token, nb = ceil(N/64).
 *  The LSE stays [B,H,N] contiguous (row b,h,i for i below sequence b's
 *  length).  Other arguments and errors as for attn_k_smooth_quant and
 *  attn_fwd_sage8; a NULL stride array is ATTN_ERR_NULL, an unknown
 *  qk_format ATTN_ERR_ARG, a misaligned cu_seqlens ATTN_ERR_ALIGN.  The
 *  preparation also takes ATTN_QK_INT8_NO_V: the INT8 Q and K of
 *  attn_k_smooth_quant bit for bit, V untouched (a workspace for
 *  attn_fwd_sage8_pv16, which reads no FP8 V; the forward here rejects that
 *  format with ATTN_ERR_ARG).
 */
attn_status attn_k_smooth_quant_strided(const void* q, const void* k, const void* v,
                                        int in_dtype, int B, int H, int N, int d,
                                        const long long* strides, const int* cu_seqlens,
                                        int qk_format, void* workspace,
                                        size_t workspace_bytes, void* stream);
attn_status attn_fwd_sage8_strided(const void* workspace, void* o, float* lse, int B,
                                   int H, int N, int d, const long long* o_strides,
                                   const int* cu_seqlens, int causal, float scale,
                                   const float* bias, int out_dtype, int qk_format,
                                   void* stream);

/*
 * attn_bwd_workspace_size -- bytes of device workspace attn_bwd_f16/bf16
 * need for this shape (one fp32 value per query row, 256-byte rounded; 0
 * when the shape is invalid for the backward).
 */
size_t attn_bwd_workspace_size(int B, int H, int N, int d);

/*
 * attn_bwd_f16 / attn_bwd_bf16 -- gradients of the fused forward (page 3,
 * "FlashAttention", the glossary paragraph: the backward pass recomputes the
 * small intermediates from the inputs instead of storing the score matrix;
 * page 5, "SAS": the log-form gate inside the softmax is trained through
 * it).  For a loss L with dout = dL/dO, with P = exp(s - LSE) the exact
 * probabilities of the forward, D = rowsum(dout * o):
 *
 *     dv = P^T dout,  dS = P * (dout v^T - D),
 *     dq = scale * dS k,  dk = scale * dS^T q,
 *     dbias[b,h,qb,kb] = sum of dS over the 64 x 64 block (qb, kb).
 *
 *  q, k, v    [B,H,N,d] of the forward, fp16 (f16 entry) or bf16.
 *  o, lse     the forward's output and its LSE (fp32).  o_dtype is q's dtype
 *             or ATTN_DTYPE_F32.  D is computed from o: with o rounded to
 *             16 bits each row of dS sums to a small rounding residue
 *             (below 2^-9 * sum |dout * o| relative to 0) instead of 0, which
 *             shows in dbias; an fp32 o removes it.
 *  dout       [B,H,N,d] dL/dO, same dtype as q.
 *  dq, dk, dv [B,H,N,d] outputs in grad_dtype: the input dtype or
 *             ATTN_DTYPE_F32.  Fully overwritten.
 *  dbias      nullable fp32 [B,H,nb,nb], nb = ceil(N/64): the gradient of
 *             the block bias (also defined when bias is NULL, as the
 *             gradient at bias = 0).  Fully overwritten.  With a bias or
 *             dbias, nb is bounded as for the forward's bias.
 *  causal, scale, bias  as passed to the forward.
 *  workspace  device buffer of at least attn_bwd_workspace_size bytes,
 *             256-byte aligned; overwritten.
 *  d must be 64, 96 or 128.  Products run on the matrix cores with fp32
 *  accumulation; P and dS are rounded to the input dtype for the products
 *  that use them.  Rows with LSE = -inf (no visible key) pass no gradient.
 *  dbias is accumulated with at most two atomic additions per element onto
 *  zero, so results are identical from run to run.
 */
attn_status attn_bwd_f16(const void* q, const void* k, const void* v, const void* o,
                         int o_dtype, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         float* dbias, int B, int H, int N, int d, int causal, float scale,
                         const float* bias, int grad_dtype, void* workspace,
                         size_t workspace_bytes, void* stream);
attn_status attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                          int o_dtype, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          float* dbias, int B, int H, int N, int d, int causal, float scale,
                          const float* bias, int grad_dtype, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * attn_bwd_noalloc -- attn_bwd_f16 / attn_bwd_bf16 (in_dtype ATTN_DTYPE_F16
 * or ATTN_DTYPE_BF16) for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The backward's scratch (one fp32 per query row) comes from a
 * fixed device array inside the library instead of a workspace argument:
 * ATTN_BWD_NOALLOC_MAX_ROWS rows (16 MiB), one copy per GPU, held until the
 * process ends.  B*H*N above that limit is ATTN_ERR_WORKSPACE.  The call
 * allocates nothing (the array's device address is looked up once per
 * device, on the first call with that device current).  Every call on one
 * GPU shares its array: calls that overlap on one GPU (different streams or
 * host threads without ordering) race and must not be issued.  Other
 * arguments, results and errors as attn_bwd_f16 / attn_bwd_bf16, which it
 * matches bit for bit.
 */
#define ATTN_BWD_NOALLOC_MAX_ROWS 4194304
attn_status attn_bwd_noalloc(int in_dtype, const void* q, const void* k, const void* v,
                             const void* o, int o_dtype, const void* dout, const float* lse,
                             void* dq, void* dk, void* dv, float* dbias, int B, int H, int N,
                             int d, int causal, float scale, const float* bias, int grad_dtype,
                             void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* attn_status_str(int status);

/* ATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
