/* libfa: fused tiled attention for AMD MI355X (gfx950).
 *
 * Computes O = Softmax(Q K^T * scale + atten_mask + pse) V and its gradients.
 *
 * The operation is the one defined in the FlashAttentionScore replacement
 * guide (jianzhnie.github.io, "FlashAttentionScore fused-op replacement"):
 * section 2 gives the formula Softmax(QK^T / sqrt(d_k)) V and states that the
 * fused operator tiles the work with an online softmax, never storing the
 * N x N score matrix, and also returns gradients with O(N) extra memory;
 * section 3.1 gives the call shape (query, key, value, head_num,
 * input_layout, pse, padding_mask, atten_mask, scale, keep_prob); section 3.2
 * the parameter meanings (layouts BSH/BNSD, key/value aligned with query,
 * pse may be ALiBi, the mask may be causal, scale is 1/sqrt(d_k), keep_prob
 * defaults to 1 = no dropout); section 4 step 1 the unfused order: scores
 * are scaled, then the additive mask is added, then softmax, then times V.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensor pointers (q, k, v, o, lse, dout, dq, dk, dv, workspace and the mask
 * and bias arrays inside fa_problem) are DEVICE pointers owned by the caller.
 * The fa_problem struct itself is host memory read only during the call.
 * The library allocates no device memory; the backward takes a caller
 * workspace of fa_bwd_workspace_size() bytes (fa_bwd_noalloc instead uses a
 * fixed device array inside the library).
 *
 * Layouts (element strides; the last dimension is contiguous):
 *   FA_BNSD: Q/O/dO/dQ [B, H, S_q, D]; K/V/dK/dV [B, H, S_k, D].
 *   FA_BSH : Q/O/dO/dQ [B, S_q, H*D]; K/V/dK/dV [B, S_k, H*D]; head h owns
 *            columns [h*D, (h+1)*D), the head split view(B,N,H,D).transpose
 *            of the multimodal page's cross-modal attention module.
 * All of Q, K, V, O, dO, dQ, dK, dV share one dtype and one layout.  LSE is
 * always float32 [B, H, S_q], natural log, and includes scale and bias.
 *
 * Masks (bits of mask_flags, combined by AND; a masked score is exactly -inf):
 *   FA_MASK_CAUSAL   key j visible to query i iff j <= i (top-left aligned
 *                    lower triangle, the ones/tril_ mask of the CogVLM guide).
 *   FA_MASK_EXPLICIT uint8 mask, nonzero = may attend, element
 *                    [b*em_stride_b + h*em_stride_h + i*em_stride_q + j];
 *                    a zero stride broadcasts that dimension (the multimodal
 *                    page's [B,N,N] bool mask expanded over heads).
 *   FA_MASK_MODALITY query i may see key j iff
 *                    modality_allow[q_modality[b,i] * M + k_modality[b,j]]
 *                    (or i == j when modality_allow_diag is set: the
 *                    multimodal page's default rule keeps the diagonal).
 *                    Modality ids are int8 in [0, M), M <= 8.
 *   FA_MASK_PADDING  key j of sample b is real iff key_valid[b*S_k + j] != 0
 *                    (the retrieval page's document mask).
 * A query row with no visible key gets O = 0, LSE = -inf, and zero gradient.
 *
 * Dropout (keep_prob < 1; the guide's section 3.2: the probability of keeping
 * an element, 1 = no dropout).  It acts on the softmax output: O = (P o M /
 * keep_prob) V, where M[b,h,i,j] = 1 iff
 *     philox4x32_10(counter = {j >> 2, i, h, b}, key = {seed & 0xffffffff,
 *                   seed >> 32}) word (j & 3)  <  floor(keep_prob * 2^32),
 * Philox4x32 with 10 rounds as published by Salmon, Moraes, Dror and Shaw
 * ("Parallel random numbers: as easy as 1, 2, 3", SC 2011), seed =
 * dropout_seed.  LSE is that of the softmax before dropout.  The backward
 * regenerates M from the same seed (no mask is stored): dV = (P o M /
 * keep_prob)^T dO, dS = P o (M o (dO V^T) / keep_prob - delta) with
 * delta_i = sum_d dO_id O_id.  F16/BF16 only.
 *
 * Gradient precision (page 1, tuning section: forward in 16 bits, backward in
 * 32): with grad_f32 set, dQ, dK and dV are written as float32 (layout of
 * Q/K/V, 16-byte aligned) instead of the input dtype.  They are the same
 * float32 values the kernels would otherwise round to 16 bits: the products
 * still take their operands (P, dS, inputs) in the input dtype with float32
 * accumulation.  Ignored for FA_F32 inputs, whose gradients are float32.
 *
 * Bias gradient (a learnable dense pse): when dpse is non-null, fa_bwd /
 * fa_bwd_main also write dpse[b, h, i, j] = dL/d(bias_ij) = dS_ij, the
 * gradient of the softmax's input (with dropout, dS_ij = P_ij (Z_ij dP_ij -
 * delta_i)); float32, contiguous [B, H, S_q, S_k], 16-byte aligned, every
 * element written (0 where the mask hides the pair).  Only with
 * pse_kind == FA_PSE_DENSE and F16/BF16 inputs; the dense bias may still be
 * broadcast in the forward, the gradient is per (b, h).
 *
 * Bias (pse, added after scaling, never scaled itself):
 *   FA_PSE_ALIBI  bias(h,i,j) = -alibi_slopes[h] * |i - j|, slopes float32 [H].
 *   FA_PSE_DENSE  bias element [b*pse_stride_b + h*pse_stride_h +
 *                 i*pse_stride_q + j] of dtype pse_dtype (F32, F16 or BF16).
 *
 * Errors: every check runs before any launch; a call that fails validation
 * writes nothing.  FA_ERR_INVALID_ARG: null pointer where one is needed,
 * negative sizes, H*D mismatch, M out of range, bad enum,
 * keep_prob outside (0, 1], reserved0 != 0, dpse set without a dense pse or
 * misaligned.  FA_ERR_UNSUPPORTED: scale < 0 (the kernels take a row's
 * maximum over raw scores before scaling), keep_prob < 1 with F32 or fp8,
 * dpse with F32 or fp8, a
 * head_dim the kernels do not cover (F16/BF16: 64 or 128; F32: 32, 64 or
 * 128), sizes past the kernels' 32-bit counters (B*H or H*D above
 * 2^31 - 1, one (batch, head) span of Q- or K-shaped rows of 2 GiB or more,
 * B*H*S_q above 2^31 - 1 rows).  FA_ERR_WORKSPACE: workspace
 * too small.  FA_ERR_HIP: a HIP launch reported an error.
 * Sizes of zero are allowed: B or H == 0 is a no-op; S_q == 0 makes the
 * forward and the steps other than fa_bwd_main a no-op, while fa_bwd and
 * fa_bwd_main write dK = dV = 0 (no query sees a key; only dk and dv are
 * read then); S_k == 0 makes every row masked (O = 0, LSE = -inf, dQ = 0).
 *
 * Synchronisation: calls enqueue work on `stream` and return without waiting.
 * Outputs are valid once the stream reaches that point.  The library keeps
 * no mutable global state; calls are thread-safe.  Two calls that write the
 * same buffers on different streams race, as with any stream work.
 *
 * Environment (read at every call; for diagnostics and sweeps): FA_LOG=1
 * prints each launch's kernel instance and grid on stderr; FA_TILE=auto
 * (default) | short | wg4 | wg1 picks the workgroup shape: wg4 and wg1 turn
 * off the kernels for short query blocks (S_q <= 32).  Results agree with
 * the definition either way, to rounding order.
 */
#ifndef LIBFA_FA_H
#define LIBFA_FA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 6

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1,
  FA_ERR_UNSUPPORTED = -2,
  FA_ERR_HIP = -3,
  FA_ERR_WORKSPACE = -4
} fa_status;

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2, FA_FP8_E4M3 = 3 } fa_dtype;
typedef enum { FA_BNSD = 0, FA_BSH = 1 } fa_layout;
enum {
  FA_MASK_NONE = 0,
  FA_MASK_CAUSAL = 1,
  FA_MASK_EXPLICIT = 2,
  FA_MASK_MODALITY = 4,
  FA_MASK_PADDING = 8
};
typedef enum { FA_PSE_NONE = 0, FA_PSE_ALIBI = 1, FA_PSE_DENSE = 2 } fa_pse_kind;

/* One attention problem.  Field order is part of the ABI (ctypes mirrors it). */
typedef struct fa_problem {
  int32_t batch;            /* B */
  int32_t head_num;         /* H (head_num of the guide's section 3.1) */
  int32_t seq_q;            /* S_q */
  int32_t seq_k;            /* S_k */
  int32_t head_dim;         /* D; for FA_BSH the hidden size is H*D */
  int32_t layout;           /* fa_layout */
  int32_t dtype;            /* fa_dtype of Q, K, V, O, dO, dQ, dK, dV */
  float scale;              /* multiplies Q K^T; no default (1/sqrt(D) is usual) */
  float keep_prob;          /* (0, 1]; < 1 applies dropout (see above) */
  uint32_t mask_flags;      /* OR of FA_MASK_* */
  int32_t num_modalities;   /* M, 1..8, for FA_MASK_MODALITY */
  int32_t modality_allow_diag; /* nonzero: i == j is always allowed */
  uint8_t modality_allow[64];  /* allow[mq * M + mk], nonzero = allowed */
  int32_t pse_kind;         /* fa_pse_kind */
  int32_t pse_dtype;        /* fa_dtype of the dense bias */
  const uint8_t *explicit_mask;      /* FA_MASK_EXPLICIT */
  int64_t em_stride_b, em_stride_h, em_stride_q;
  const int8_t *q_modality;          /* [B, S_q] */
  const int8_t *k_modality;          /* [B, S_k] */
  const uint8_t *key_valid;          /* [B, S_k] */
  const float *alibi_slopes;         /* [H] */
  const void *pse;                   /* dense bias */
  int64_t pse_stride_b, pse_stride_h, pse_stride_q;
  uint64_t dropout_seed;             /* Philox key when keep_prob < 1 */
  int32_t grad_f32;                  /* nonzero: the backward writes dQ, dK, dV as float32 */
  int32_t reserved0;                 /* must be 0 */
  float *dpse;                       /* optional backward output, see "Bias gradient" */
} fa_problem;

/* Forward: O (layout/dtype of Q) and LSE (float32 [B,H,S_q]). */
fa_status fa_fwd(const fa_problem *p, const void *q, const void *k, const void *v,
                 void *o, float *lse, hipStream_t stream);

/* Forward with fp8 inputs (page 1, tuning section: pure fp8, experimental).
 * p->dtype must be FA_FP8_E4M3: q, k, v hold OCP e4m3 bytes (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits; no infinities; the value of a
 * byte times its tensor's descale factor is the real input; the three
 * descale factors must be finite and positive).  O is bf16 in
 * Q's layout, LSE float32 [B,H,S_q], both as for fa_fwd, for the real inputs.
 * Masks and bias as for fa_fwd; D = 64 or 128; keep_prob must be 1.
 * The probabilities that multiply V are rounded to e4m3 (p = exp2 of the
 * logit minus a running reference, at most 2^8); the row sums use them
 * unrounded.  The workspace (fa_fwd_fp8_workspace_size bytes, 16-byte
 * aligned) receives V transposed per 64-key tile; it needs no clearing.
 * fa_fwd, fa_bwd* reject FA_FP8_E4M3 with FA_ERR_UNSUPPORTED. */
fa_status fa_fwd_fp8_workspace_size(const fa_problem *p, size_t *bytes);
fa_status fa_fwd_fp8(const fa_problem *p, const void *q, const void *k, const void *v,
                     float q_descale, float k_descale, float v_descale, void *o, float *lse,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace fa_bwd needs: the float32 row terms
 * D_i = sum_d dO_id * O_id, [B,H,S_q], rounded up to 256 bytes. */
fa_status fa_bwd_workspace_size(const fa_problem *p, size_t *bytes);

/* Backward: given Q, K, V, the forward's O and LSE and the upstream dO,
 * writes dQ, dK, dV (layout/dtype of Q/K/V) of L = sum(O * dO).  P is
 * recomputed tile by tile from LSE (guide section 2: gradients without the
 * N x N matrix).  No atomics are used: the result is bitwise repeatable.
 * fa_bwd is exactly the sequence of the three steps below on `stream`. */
fa_status fa_bwd(const fa_problem *p, const void *q, const void *k, const void *v,
                 const void *o, const float *lse, const void *dout,
                 void *dq, void *dk, void *dv,
                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, outputs and errors as fa_bwd minus the
 * workspace: the row terms D_i live in a static device array of
 * FA_NOALLOC_SCRATCH_BYTES bytes inside the library (one per GPU, held until
 * the process ends), so the problem must satisfy
 * 4 * B * H * S_q <= FA_NOALLOC_SCRATCH_BYTES (rounded up to 256 bytes),
 * else FA_ERR_WORKSPACE, before any launch.  The call allocates nothing.
 * The stream must belong to the current device; the array's address there is
 * looked up once per device (FA_ERR_HIP if that fails).  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams, other
 * host threads) race and give wrong gradients; calls ordered on one stream do
 * not.  The array needs no clearing: each call writes the row terms it reads. */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
fa_status fa_bwd_noalloc(const fa_problem *p, const void *q, const void *k, const void *v,
                         const void *o, const float *lse, const void *dout,
                         void *dq, void *dk, void *dv, hipStream_t stream);

/* Backward step 1: row terms D_i = sum_d dO_id * O_id into the workspace. */
fa_status fa_bwd_prep(const fa_problem *p, const void *o, const void *dout,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward step 2 (key-tile pass): for each key tile, recompute P and dS over
 * the query tiles that see it and write dV = P^T dO and dK = scale dS^T Q.
 * Reads the row terms of step 1 from the workspace. */
fa_status fa_bwd_main(const fa_problem *p, const void *q, const void *k, const void *v,
                      const float *lse, const void *dout, void *dk, void *dv,
                      const void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward step 3 (query-tile pass): for each query tile, recompute P and dS
 * over the key tiles it sees and write dQ = scale dS K.  Reads the row terms
 * of step 1 from the workspace; independent of step 2. */
fa_status fa_bwd_post(const fa_problem *p, const void *q, const void *k, const void *v,
                      const float *lse, const void *dout, void *dq,
                      const void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * MaxSim late-interaction score (retrieval page, "Layer 2: semantic
 * modelling"): for sample b, the similarity of query token i and document
 * token j is the plain dot product sim_ij = q_i . d_j over the embedding
 * width (no scale, no softmax).  Invalid document tokens are excluded
 * (-inf); each query token keeps its best match, rowmax_i = max_j sim_ij; the
 * score is the sum of rowmax over the valid query tokens divided by L_q.
 *
 *   q [B, L_q, D], d [B, L_d, D]: contiguous rows, dtype FA_BF16 or FA_F16,
 *       device pointers, 16-byte aligned (d may be NULL when L_d == 0);
 *   q_valid [B, L_q], d_valid [B, L_d]: uint8, nonzero = real token; NULL
 *       means every token is real;
 *   rowmax float32 [B, L_q] (may be NULL when L_q == 0): -inf for an invalid
 *       query token and for a query token with no valid document token;
 *   score float32 [B] (may be NULL when B == 0): the sum over valid query
 *       tokens of rowmax, divided by L_q; 0 when no query token is valid
 *       (including L_q == 0); -inf when a valid query token sees no valid
 *       document token.
 *
 * The dot products are accumulated in float32 from exact products; the
 * result is bitwise repeatable.  Errors: FA_ERR_INVALID_ARG for a null
 * struct, negative sizes, a bad dtype enum, pad0 != 0, or a
 * missing/misaligned tensor; FA_ERR_UNSUPPORTED for FA_F32, D not a multiple
 * of 128 or above 1024, or L_d above 16384.  B == 0 is a no-op.
 * Synchronisation as for the attention entry points; no workspace.
 * ------------------------------------------------------------------------ */
typedef struct fa_maxsim_problem {
  int32_t batch;            /* B */
  int32_t len_q;            /* L_q */
  int32_t len_d;            /* L_d */
  int32_t dim;              /* D, the embedding width */
  int32_t dtype;            /* fa_dtype of q and d */
  int32_t pad0;             /* must be 0 */
  const uint8_t *q_valid;   /* [B, L_q] or NULL */
  const uint8_t *d_valid;   /* [B, L_d] or NULL */
} fa_maxsim_problem;

fa_status fa_maxsim(const fa_maxsim_problem *p, const void *q, const void *d, float *rowmax,
                    float *score, hipStream_t stream);

const char *fa_status_str(fa_status s);
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBFA_FA_H */
