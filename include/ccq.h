/*
 * ccq.h -- C ABI of the MI355X (gfx950) Curvature-Conditioned Query read step.
 *
 * The method (gist.science summary of arXiv 2606.01294, "不要阅读一切：一种基于曲率条件
 * 的线性注意力查询", §2 "理论推导", "机制" and "集成"):
 *   keys are unit vectors; the running, undecayed key statistics give
 *     mu_t = (1/t) sum_{j<=t} k_j,  Cbar_t = (1/t) sum_{j<=t} k_j k_j^T,
 *     Sigma_t = Cbar_t - mu_t mu_t^T;
 *   the gate is lambda_t = sigmoid(w_lambda . q_t + b_lambda) (one scalar per token and head);
 *   the cleaned query is q_clean = q_t - lambda_t Sigma_t q_t;
 *   the write rule is left as it is, and the read is o_t = S_t q_clean with S_t the
 *   state after token t's write.
 * Write rules (named by the pages, standard definitions):
 *   CCQ_RULE_GLA : S_t = S_{t-1} diag(alpha_t) + v_t k_t^T,  alpha_t = exp(log_alpha_t) per key channel;
 *   CCQ_RULE_GDN : S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, scalar alpha_t, beta_t.
 *
 * Statistic state.  The pages keep one extra d_k x d_k matrix and one d_k vector per head
 * (summary §2 "机制").  This library stores them as SUMS: C = sum k k^T, ksum = sum k, plus
 * the token count n, and applies 1/n per token.
 *
 * Conventions for every entry point
 *   - All pointers are DEVICE pointers owned by the caller; the library allocates no memory,
 *     keeps no pointer after it returns and holds no global mutable state.  Calls are
 *     reentrant.  The one exception is ccq_fwd_chunked_noalloc, whose workspace is a device
 *     array the library holds (see there).
 *   - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the default stream) without any
 *     host synchronisation.  The caller keeps buffers alive until the stream has passed the
 *     call.
 *   - Every pointer must be 16-byte aligned.  Tensors are dense, row-major, in the shapes
 *     given below.
 *   - Argument errors return a negative ccq_status BEFORE anything is enqueued.  A failed
 *     launch returns CCQ_ERR_LAUNCH.  Faults inside a kernel surface at the caller's next
 *     synchronisation; the library does not hide them.
 *   - Keys must be L2-normalised (unit keys are the precondition of the eigenvalue bound
 *     eig(I - lambda Sigma) in [1 - lambda, 1], 10100.com write-up, section "方法解析"): either
 *     by the caller, or by the library when CCQ_FLAG_NORMALIZE_KEYS is set.
 *   - Supported shapes: d_k == d_v, d in {64, 128} for CCQ_DTYPE_BF16, d == 64 for
 *     CCQ_DTYPE_F32; chunk == 64 (or 0, meaning 64).  Anything else is CCQ_ERR_UNSUPPORTED.
 */
#ifndef CCQ_H_
#define CCQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CCQ_OK = 0,
  CCQ_ERR_INVALID_ARG = -1,  /* null required pointer, non-positive size, bad enum, partial carry */
  CCQ_ERR_UNSUPPORTED = -2,  /* valid request this build has no kernel for (d, dtype, chunk)    */
  CCQ_ERR_MISALIGNED = -3,   /* a pointer is not 16-byte aligned                                 */
  CCQ_ERR_LAUNCH = -4,       /* the HIP runtime refused a launch                                 */
  CCQ_ERR_WORKSPACE = -5     /* workspace missing or smaller than ccq_fwd_workspace_bytes()      */
} ccq_status;

typedef enum { CCQ_RULE_GLA = 0, CCQ_RULE_GDN = 1 } ccq_rule;

/* Storage dtype of q, k, v, log_alpha, beta and o.  The carry is always fp32. */
typedef enum { CCQ_DTYPE_F32 = 0, CCQ_DTYPE_BF16 = 1 } ccq_dtype;

/* Option bits (ccq_fwd_params.flags, ccq_decode_step's flags).
 * CCQ_FLAG_NORMALIZE_KEYS: the library scales every key to unit L2 norm, k / max(|k|, 1e-12)
 * computed in fp32 from the stored key, before any use (statistics, gate, read and write).
 * Without it keys are used as given and must already be unit vectors.
 * CCQ_FLAG_PACKED_COV: the second-moment sum C, which is symmetric, is passed as its upper
 * triangle only: d_k (d_k + 1) / 2 fp32 entries per head, row by row (C[0][0..d_k-1],
 * C[1][1..d_k-1], ..., C[d_k-1][d_k-1]), so entry C[i][j], i <= j, sits at index
 * i d_k - i (i - 1) / 2 + (j - i).  It applies to C0 and C_out of ccq_fwd_chunked and to C
 * of ccq_decode_step, whose per-head stride becomes d_k (d_k + 1) / 2.  The statistics
 * are the extra state the method keeps per head (summary §2 "机制"); the 10100.com
 * write-up's section "代价与边界" names that state's memory as the method's inference cost,
 * and the packed form moves about half of C's bytes in a decode step. */
typedef enum { CCQ_FLAG_NORMALIZE_KEYS = 1, CCQ_FLAG_PACKED_COV = 2 } ccq_flag;

/* Arguments of ccq_fwd_chunked.  Zero-initialise, then fill in. */
typedef struct {
  int32_t rule;   /* ccq_rule  */
  int32_t dtype;  /* ccq_dtype */
  int32_t B, H, T;
  int32_t d_k, d_v;
  int32_t chunk;     /* 64, or 0 for the default (64)                                         */
  int32_t segments;  /* sequence segments per (b, h) chain processed in parallel; 0 = choose  */

  const void *q;         /* [B, H, T, d_k] dtype                                               */
  const void *k;         /* [B, H, T, d_k] dtype, unit rows                                    */
  const void *v;         /* [B, H, T, d_v] dtype                                               */
  const void *log_alpha; /* GLA: [B, H, T, d_k]; GDN: [B, H, T]; dtype; log of the decay       */
  const void *beta;      /* GDN: [B, H, T] dtype in (0, 1); GLA: must be NULL                  */
  const float *w_lambda; /* [H, d_k] fp32 gate weights                                          */
  const float *b_lambda; /* [H] fp32 gate bias (-INFINITY switches the cleaning off exactly)    */

  /* Carry in: all four NULL (start from zeros, n0 = 0) or all four set. */
  const float *S0;       /* [B, H, d_v, d_k]                                                    */
  const float *C0;       /* [B, H, d_k, d_k]  sum of k k^T  ([B, H, d_k (d_k+1)/2] packed)      */
  const float *ksum0;    /* [B, H, d_k]       sum of k                                          */
  const int64_t *n0;     /* [B, H]            token count                                       */

  void *o;               /* [B, H, T, d_v] dtype, written                                       */

  /* Carry out: all four NULL (not wanted) or all four set.  May alias or overlap the carry in:
   * with more than one segment the call then first copies the carry in (and n0) into the
   * workspace, which ccq_fwd_workspace_bytes always leaves room for, and reads only the copy. */
  float *S_out;
  float *C_out;          /* same layout as C0                                                    */
  float *ksum_out;
  int64_t *n_out;

  void *workspace;        /* device scratch of at least ccq_fwd_workspace_bytes(p) bytes, or  */
  size_t workspace_bytes; /* NULL / 0 when that function returns 0                            */

  /* Optional per-kernel timing: NULL, or an array of 4 caller-created hipEvent_t that are
   * recorded on hip_stream before the segment-summary kernel, after it, after the carry scan
   * and after the main kernel.  With one segment the first three are recorded together,
   * just before the main kernel.  A failed record returns CCQ_ERR_LAUNCH. */
  void *const *phase_events;

  int32_t flags;          /* ccq_flag bits; unknown bits are CCQ_ERR_INVALID_ARG            */

  /* Optional (training): NULL, or ccq_chunk_carry_bytes(dtype, B, H, T, d_k) bytes of device
   * memory that receive the carry at the start of every 64-token chunk c of every chain
   * i = b H + h, for a later ccq_bwd_chunked of the same inputs (its chunk_carry): S_c then C_c,
   * each [d][d] row-major in dtype, at element offset (i NC + c) 2 d^2 (NC = ceil(T / 64); C full,
   * whatever the flags say about the carry in and out), followed by the key sums m_c, [d] fp32
   * each, at float offset (i NC + c) d of the region after all of them.  The chunk carries are
   * those of the keys as used (normalised in the kernel if the flag asks for it).  16-byte
   * aligned (else CCQ_ERR_MISALIGNED). */
  void *chunk_carry;
} ccq_fwd_params;

/* Bytes of the chunk-carry buffer of ccq_fwd_params.chunk_carry / ccq_bwd_params.chunk_carry for
 * these sizes (0 for an unsupported dtype, non-positive sizes or d_k != d_v shapes the chunked
 * calls reject): B H ceil(T / 64) (2 d^2 sizeof(dtype) + 4 d). */
size_t ccq_chunk_carry_bytes(int32_t dtype, int32_t B, int32_t H, int32_t T, int32_t d);

/*
 * Chunked prefill of one CCQ layer: o for every token and, optionally, the final carry.
 * The result is the per-token recurrence above evaluated exactly (up to rounding) with
 * chunks of 64 tokens; the statistics are carried chunk by chunk exactly as the backbone's
 * state is (summary §2 "机制").  A call with a carry in continues the sequence
 * the carry came from.  T need not be a multiple of 64.
 * Precondition (GLA): the call cuts its T tokens into chunks of 64 counted from its own first
 * token (tokens 64c .. 64c + 63).  Within every chunk the decay is factored with the chunk's
 * start as reference, so for every key channel the sum of log_alpha over a whole chunk
 * (equivalently, since log_alpha <= 0, from the chunk's first token to any later token of it)
 * must stay above -80: an average log decay above -1.25 per token (alpha > 0.29).  Beyond it
 * e^{-B} overflows in fp32 and o and the carry are not finite; nothing checks this.
 * Gated DeltaNet has no such limit.  Returns a ccq_status.
 */
int ccq_fwd_chunked(const ccq_fwd_params *p, void *hip_stream);

/* Bytes of device workspace ccq_fwd_chunked needs for these arguments (0 if none).  Depends
 * only on rule, dtype, B, H, T, d_k, d_v, chunk and segments.  Returns 0 for invalid p too. */
size_t ccq_fwd_workspace_bytes(const ccq_fwd_params *p);

/* Size of the device array ccq_fwd_chunked_noalloc takes its workspace from: 64 MiB. */
#define CCQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * ccq_fwd_chunked for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It computes exactly what
 * ccq_fwd_chunked computes, with the same kernels, but calls no allocating routine and takes no
 * workspace: p->workspace and p->workspace_bytes are ignored, and the workspace is a
 * CCQ_NOALLOC_SCRATCH_BYTES device array inside the library.  Each device the library runs on
 * holds its own copy of that array from the first such call on it until the process ends.
 * Segments: with p->segments == 0 the library's own choice, made longer (fewer per chain) until
 * its workspace fits the array; a p->segments whose workspace (ccq_fwd_workspace_bytes) exceeds
 * CCQ_NOALLOC_SCRATCH_BYTES returns CCQ_ERR_WORKSPACE before anything is enqueued.  Every call
 * on a device shares that device's array and leaves its contents behind (no call needs it to
 * start at zero): calls that can overlap on one device -- on different streams, or from
 * different threads -- race on it and must be serialised by the caller.  The first call on a
 * device looks the array up (hipGetSymbolAddress) with that device current; a failed lookup
 * returns CCQ_ERR_LAUNCH.  Other arguments, errors and semantics as ccq_fwd_chunked.
 */
int ccq_fwd_chunked_noalloc(const ccq_fwd_params *p, void *hip_stream);

/*
 * One decode step for N sequences x H heads, state updated in place:
 *   n += 1; C += k k^T; ksum += k; Sigma q = C q / n - ksum (ksum . q) / n^2;
 *   q_clean = q - lambda Sigma q; write rule; o = S q_clean.
 * q, k: [N, H, d_k] dtype; v: [N, H, d_v] dtype; log_alpha: GLA [N, H, d_k] / GDN [N, H];
 * beta: GDN [N, H] (GLA: NULL); w_lambda [H, d_k], b_lambda [H] fp32;
 * S [N, H, d_v, d_k], C [N, H, d_k, d_k] (with CCQ_FLAG_PACKED_COV: [N, H, d_k (d_k+1)/2]),
 * ksum [N, H, d_k] fp32 and n [N, H] int64 are read and written in place; o [N, H, d_v]
 * dtype is written.  flags: ccq_flag bits; unknown bits are CCQ_ERR_INVALID_ARG.
 * Returns a ccq_status.
 */
int ccq_decode_step(int32_t rule, int32_t dtype, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                    const void *q, const void *k, const void *v, const void *log_alpha,
                    const void *beta, const float *w_lambda, const float *b_lambda, float *S,
                    float *C, float *ksum, int64_t *n, void *o, int32_t flags, void *hip_stream);

/*
 * Key-covariance subspace diagnostic (the geometric check of the 10100.com write-up, section
 * "记忆体检": Δμ, how much less needle keys than distractor keys align with the top-16
 * eigen-subspace of the key covariance; negative means the needle lies off the high-variance
 * directions).  Per (b, h):
 *   Sigma = C / n - mu mu^T with mu = ksum / n (the statistics of the read step; C, ksum, n as
 *           carried by ccq_fwd_chunked / ccq_decode_step; n <= 0 gives Sigma = 0),
 *   eigvals [B, H, d_k]    : the eigenvalues of Sigma, descending,
 *   basis   [B, H, r, d_k] : the top-r unit eigenvectors as rows, each with its largest-
 *                            magnitude entry positive (the lowest index among equal ones),
 *   align   [B, H, T]      : a_t = |basis k_t|^2 / |k_t|^2 for every key k_t of k
 *                            ([B, H, T, d_k] dtype; a_t = 0 for a zero key),
 *   delta_mu [B, H]        : mean a_t over tokens with needle[b][h][t] != 0 minus the mean over
 *                            the others (NaN when either set is empty); needle [B, H, T] uint8,
 *   iters   [B, H] int32   : bisection work of the head: the multisection rounds of its d_k
 *                            eigenvalues, summed (0 for Sigma = 0; optional, may be NULL).
 * needle and delta_mu are both NULL (no Δμ) or both set; iters may be NULL; every other
 * pointer is required.
 * flags: CCQ_FLAG_PACKED_COV (C packed as for the other entry points); other bits are
 * CCQ_ERR_INVALID_ARG.  1 <= r <= min(32, d_k); d_k in {64, 128}; B * H <= 65535; dtype as for
 * the other entry points.  The eigen-decomposition runs in fp32: Householder tridiagonalisation,
 * bisection on Sturm counts for the eigenvalues (to about 1e-6 of the largest), inverse
 * iteration with Gram-Schmidt for the eigenvectors (orthonormal to about 1e-6); the subspace, and with it a_t, is well defined when eigenvalue r
 * exceeds eigenvalue r + 1.  Returns a ccq_status.
 */
int ccq_key_subspace(int32_t dtype, int32_t B, int32_t H, int32_t T, int32_t d_k, int32_t r,
                     const float *C, const float *ksum, const int64_t *n, const void *k,
                     const uint8_t *needle, float *eigvals, float *basis, float *align,
                     float *delta_mu, int32_t *iters, int32_t flags, void *hip_stream);

/*
 * Backward of one step of the recurrence (the adjoint of ccq_decode_step), for training: the
 * pages train CCQ models from scratch (10100.com write-up, section "方法解析" point 3).  For N
 * sequences x H heads, given the carry BEFORE the step (S, C, ksum, n: as ccq_decode_step reads
 * them, full-matrix C), the token (q, k, v, log_alpha, beta), the gate parameters, the output
 * gradient d_o [N, H, d_v] fp32 and the adjoint of the carry AFTER the step (dS [N, H, d_v, d_k],
 * dC [N, H, d_k, d_k], dksum [N, H, d_k], fp32; zeros after the last token), it
 *   - overwrites dS, dC, dksum in place with the adjoint of the carry BEFORE the step (dC is
 *     the adjoint of C as a general matrix; only its symmetric part acts on keys),
 *   - writes the fp32 gradients dq, dk [N, H, d_k], dv [N, H, d_v], dlog_alpha (GLA [N, H, d_k],
 *     GDN [N, H]), dbeta (GDN [N, H]; GLA: NULL), and per-sequence gate-parameter gradients
 *     dw_lambda [N, H, d_k] and db_lambda [N, H] (the gradient of the shared [H, d_k] / [H]
 *     parameters is their sum over sequences and steps).
 * Running it over the tokens of a sequence in reverse order, each time from that token's carry
 * before the step, gives the gradients of the whole recurrence (backpropagation through time).
 * Inputs are used as given (flags must be 0: no in-kernel key normalisation, full C).
 * d_k == d_v == 128; dtype is that of q, k, v, log_alpha, beta.  Returns a ccq_status.
 */
int ccq_step_backward(int32_t rule, int32_t dtype, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                      const void *q, const void *k, const void *v, const void *log_alpha,
                      const void *beta, const float *w_lambda, const float *b_lambda,
                      const float *S, const float *C, const float *ksum, const int64_t *n,
                      const float *d_o, float *dS, float *dC, float *dksum, float *dq, float *dk,
                      float *dv, float *dlog_alpha, float *dbeta, float *dw_lambda,
                      float *db_lambda, int32_t flags, void *hip_stream);

/* Static description of a status code (never NULL). */
const char *ccq_status_string(int32_t status);

/* ABI version of this header: 10. */
int32_t ccq_abi_version(void);

/* Arguments of ccq_bwd_chunked.  Zero-initialise, then fill in. */
typedef struct {
  int32_t rule;   /* ccq_rule: CCQ_RULE_GLA or CCQ_RULE_GDN                                      */
  int32_t dtype;  /* ccq_dtype of q, k, v, log_alpha and d_o                                       */
  int32_t B, H, T;
  int32_t d_k, d_v;
  int32_t chunk;  /* 64, or 0 for the default (64)                                                 */

  /* The forward's inputs, exactly as given to ccq_fwd_chunked (unit keys, no flags); log_alpha is
   * [B, H, T, d_k] for GLA and [B, H, T] for Gated DeltaNet (whose beta comes at the end). */
  const void *q, *k, *v, *log_alpha; /* [B, H, T, d] dtype                                         */
  const float *w_lambda;             /* [H, d_k]                                                    */
  const float *b_lambda;             /* [H]                                                         */
  const float *S0, *C0, *ksum0;      /* carry in: all four NULL (zeros) or all four set (full C)    */
  const int64_t *n0;

  const void *d_o;                   /* [B, H, T, d_v] dtype: gradient of the loss w.r.t. o          */
  /* Adjoint of the carry out (gradient of the loss w.r.t. S_T, C_T, ksum_T): all NULL (zero) or
   * all set; [B, H, d_v, d_k], [B, H, d_k, d_k] (as a general matrix), [B, H, d_k] fp32. */
  const float *dS_T, *dC_T, *dksum_T;

  /* Gradients, fp32, written: */
  float *dq, *dk;        /* [B, H, T, d_k]                                                          */
  float *dv;             /* [B, H, T, d_v]                                                          */
  float *dlog_alpha;     /* [B, H, T, d_k] (GLA) or [B, H, T] (Gated DeltaNet)                      */
  float *dw_lambda;      /* [B, H, d_k] per sequence: the [H, d_k] parameter's gradient is their sum */
  float *db_lambda;      /* [B, H]      per sequence                                                */
  float *dS0, *dC0, *dksum0; /* adjoint of the carry in: all NULL (not wanted) or all set          */

  void *workspace;        /* at least ccq_bwd_workspace_bytes(p) bytes of device memory             */
  size_t workspace_bytes;
  /* Optional per-pass timing: NULL, or 5 caller-created hipEvent_t recorded before the chunk
   * carries, after them, after pass A, after the reverse scan and after pass B. */
  void *const *phase_events;
  int32_t flags;          /* must be 0                                                               */
  /* Gated DeltaNet only (both NULL for GLA): the forward's beta [B, H, T] (dtype) and its
   * gradient dbeta [B, H, T] (fp32, written). */
  const void *beta;
  float *dbeta;
  /* Optional: NULL (the backward recomputes the forward carry at every chunk start), or the
   * chunk_carry buffer a ccq_fwd_chunked call with the same inputs and carry in filled (layout
   * there); the backward then reads the chunk carries from it and skips their recomputation
   * (the segment summary, scan and chunk walk).  Results agree with the recomputing path up to
   * rounding.  16-byte aligned (else CCQ_ERR_MISALIGNED). */
  const void *chunk_carry;
} ccq_bwd_params;

/*
 * Chunked backward of ccq_fwd_chunked, on either write rule (training; the pages train CCQ models
 * on both backbones from scratch, 10100.com write-up, section "方法解析" point 3, gist.science
 * summary §4): for the loss
 *   L = <d_o, o> + <dS_T, S_T> + <dC_T, C_T> + <dksum_T, ksum_T>
 * of the forward with the same inputs and carry in, it writes dL/dq, dL/dk, dL/dv,
 * dL/dlog_alpha (and dL/dbeta for Gated DeltaNet), the per-sequence gate-parameter gradients and,
 * when asked for, the adjoint of the carry in.  The forward carry at every 64-token chunk start is
 * recomputed, or read from the forward's chunk_carry when given, and each chunk's gradients follow from it and the
 * adjoint carried back from later chunks: for GLA through the diagonal decay, for Gated DeltaNet
 * through the transpose of each chunk's d_k x d_k state transition.  Results equal
 * backpropagation through the per-token recurrence up to rounding; the forward's precondition on
 * the GLA log decay applies.
 * Supported: d_k == d_v, d in {64, 128} for CCQ_DTYPE_BF16, d == 64 for CCQ_DTYPE_F32,
 * flags == 0; B * H <= 65535; B * H * ceil(T / 64) < 2^31.  beta and dbeta are set for Gated
 * DeltaNet and NULL for GLA (else CCQ_ERR_INVALID_ARG).  Returns a ccq_status.
 */
int ccq_bwd_chunked(const ccq_bwd_params *p, void *hip_stream);

/* Bytes of device workspace ccq_bwd_chunked needs (0 for invalid p).  Depends only on rule,
 * dtype, B, H, T and d_k: per (b, h) and 64-token chunk, the carry and the carried-back adjoints
 * and fp32 [64, d_k] tiles (GLA: also the forward carry update, 0.36 MB per chunk at d_k = 128,
 * bf16; Gated DeltaNet: also the chunk's 64 x 64 triangular inverse, 0.21 MB per chunk), plus for
 * Gated DeltaNet the prefill's segment slots. */
size_t ccq_bwd_workspace_bytes(const ccq_bwd_params *p);

#ifdef __cplusplus
}
#endif

#endif /* CCQ_H_ */
