/*
 * gdn.h -- C ABI of libgdn.so: the chunked gated delta rule (Gated DeltaNet) on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  Per sequence and head, with a d_k x d_v state S (initial
 * value S0, or zero) and for every token t in order:
 *
 *     S <- exp(g_t) * S                         forget
 *     e  = beta_t * (v_t - S^T k_t)             error of what is stored under k_t
 *     S <- S + k_t e^T                          write
 *     o_t = scale * S^T q_t                     read with the query, after the write
 *
 * This is the update of "Research Sprint Day 1 - Verifying the
 * flash-linear-attention Gated DeltaNet kernel on GB10", section "The GDN update",
 * with alpha = exp(g) kept in log space as on "Research Sprint Day 2 - Rooflines",
 * section "Building some intuition" (gates, step 5).  Its closed form on the
 * Day-2 page is S'_t = S'_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 * with S' = S^T.  `scale` is the query scale that the cuLA issue #126 page
 * ("Minimal public reproduction") passes to its kernels as a separate argument.
 *
 * gdn_chunk_fwd / gdn_chunk_bwd evaluate this in chunks of 64 tokens (the
 * "chunk_gated_delta_rule" of the Day-1 page, "Conclusion"; intermediates of the
 * fla issue #1550 page, "Intermediate rounding diagnosis").  gdn_recurrent_ref
 * runs the token loop itself in IEEE fp32 (the "fused recurrent operator" of the
 * fla issue #1550 page, "Reproduction and evidence").
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - Tensors are dense, row-major, last dimension contiguous, on the device:
 *      q, k              [B, T, H, Dk]     io dtype
 *      v, o, dO, dv      [B, T, H, Dv]     io dtype
 *      dq, dk            [B, T, H, Dk]     io dtype
 *      g, beta, dg, dbeta[B, T, H]         fp32
 *      S0, S_final, dS_final, dS0
 *                        [N, H, Dk, Dv]    fp32  (N = number of sequences)
 *  - Packed variable-length sequences (fla issue #1550 page: sequence lengths
 *    [5120, 5120] in one row): B must be 1 and sequence n is tokens
 *    [cu[n], cu[n+1]) of the row.  Chunks restart at every sequence start; each
 *    sequence has its own S0 / S_final.  The caller passes the offsets twice:
 *    on the host (validated before any launch) and as a device copy holding the
 *    same values (read by the kernels).  Dense input: both NULL, N = B.
 *  - The value domain is documented, not checked: g <= 0 (alpha = exp(g) in
 *    (0, 1]), beta in (0, 2) (Day-2 page: beta = 2 sigmoid(.) under
 *    allow_neg_eigval), k rows L2-normalised.  NaN and Inf propagate.
 *  - Ownership: the caller allocates every buffer, including the workspace
 *    sized by gdn_workspace_size.  The library allocates nothing, keeps no state
 *    between calls and never synchronises the host -- except
 *    gdn_chunk_fwd_noalloc, whose workspace is a fixed device array the library
 *    holds (see there).
 *  - Execution: asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Outputs are always overwritten, never accumulated.
 *  - Errors: every shape, pointer, dtype, support and workspace check happens on
 *    the host before the first launch, so an error leaves every output untouched.
 *    GDN_ERR_HIP reports a failed launch (hipGetLastError).  There is no silent
 *    fallback: an unsupported case is an error.
 *  - Precision (explicit, never switched by environment variables):
 *      io dtype GDN_FP32: every product in IEEE fp32 (fp32 MFMA), fp32 state.
 *      io dtype GDN_BF16: bf16 MFMA operands with fp32 accumulation; the state,
 *        the decay factors, the triangular solve and all gradients' reductions
 *        are fp32; outputs are rounded to bf16 (round to nearest even) once.
 *  - Supported: Dk in {64, 128};
 *    Dv a multiple of 16 with 16 <= Dv <= 256; chunk == 64; num_segments in
 *    {1, 2, 4, 8, 16}; N <= 65535.  The recurrent backward needs
 *    2 * Dk * (Dv + 1) * 4 bytes of LDS and so Dk * Dv <= 128 * 128.
 *  - All entry points are thread-safe.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 6

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL                               */
  GDN_ERR_SHAPE = 2,       /* a size is out of range or inconsistent                   */
  GDN_ERR_DTYPE = 3,       /* io_dtype is not a gdn_dtype                              */
  GDN_ERR_UNSUPPORTED = 4, /* valid but not built: Dk, Dv, chunk or num_segments       */
  GDN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than gdn_workspace_size        */
  GDN_ERR_ALIAS = 6,       /* an output overlaps an input or another output            */
  GDN_ERR_HIP = 7,         /* a HIP launch failed                                      */
  GDN_ERR_SEQLENS = 8,     /* cu_seqlens not 0 = cu[0] <= cu[1] <= ... <= cu[N] = T     */
  GDN_ERR_ALIGN = 9,       /* q, k, v, o, dO, dq, dk, dv not 16-byte aligned, or an fp32
                              tensor not 4-byte aligned                                 */
  GDN_ERR_SCRATCH = 10     /* gdn_chunk_fwd_noalloc: the problem needs more workspace than
                              GDN_NOALLOC_SCRATCH_BYTES                                 */
} gdn_status;

typedef enum gdn_dtype { GDN_FP32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Precision policy of the chunked products (the fla issue #1550 page, "Proposed
 * scope", asks for a policy for the score and WY intermediates that keeps the
 * public dtypes, chosen on measured latency and memory):
 *   GDN_PRECISION_IO   the io dtype decides: bf16 io -> bf16 MFMA operands (the
 *                      inverse T diag(beta), the score P, R, E and the state
 *                      operand rounded to bf16) with fp32 accumulation, state and
 *                      decays; fp32 io -> every product in IEEE fp32.
 *   GDN_PRECISION_FP32 every product in IEEE fp32 (fp32 MFMA) whatever the io
 *                      dtype: bf16 inputs are widened exactly, o is rounded to
 *                      bf16 once, the per-chunk workspace records are fp32.
 *                      gdn_chunk_fwd only (gdn_chunk_bwd, gdn_kda_chunk_fwd and
 *                      gdn_kda_chunk_bwd with bf16 io return GDN_ERR_UNSUPPORTED
 *                      for it). */
typedef enum gdn_precision { GDN_PRECISION_IO = 0, GDN_PRECISION_FP32 = 1 } gdn_precision;

typedef enum gdn_pass {
  GDN_PASS_CHUNK_FWD = 0,
  GDN_PASS_CHUNK_BWD = 1,
  GDN_PASS_RECURRENT_FWD = 2,
  GDN_PASS_RECURRENT_BWD = 3,
  GDN_PASS_KDA_FWD = 4,
  GDN_PASS_CHUNK_SAVED = 5, /* the buffer of gdn_chunk_fwd_save / gdn_chunk_bwd_saved */
  GDN_PASS_KDA_BWD = 6,
  GDN_PASS_KDA_SAVED = 7    /* the buffer of gdn_kda_chunk_fwd_save / gdn_kda_chunk_bwd_saved */
} gdn_pass;

typedef struct gdn_problem {
  int32_t B, T, H, Dk, Dv;         /* sizes; T may be 0                                     */
  int32_t num_seqs;                /* N: == B for dense input, else len(cu_seqlens) - 1     */
  const int32_t* cu_seqlens_host;  /* host, N + 1 offsets, or NULL (dense)                  */
  const int32_t* cu_seqlens_dev;   /* device copy of the same N + 1 values, or NULL         */
  int32_t io_dtype;                /* gdn_dtype of q, k, v, o, dO, dq, dk, dv               */
  float scale;                     /* output scale: o_t = scale * S_t^T q_t                 */
  int32_t chunk;                   /* tokens per chunk; must be 64                          */
  int32_t num_segments;            /* 1: serial over chunks; G > 1: segment split (fwd)     */
  int32_t precision;               /* gdn_precision of the chunked products                 */
} gdn_problem;

/* Version of this ABI (GDN_ABI_VERSION). */
int32_t gdn_abi_version(void);

/* Static string naming a status code; never NULL. */
const char* gdn_status_str(int32_t status);

/* Bytes of device workspace that `pass` needs for `problem` (0 is possible; the
 * workspace pointer may then be NULL).  Validates the problem like the entry
 * point it sizes for. */
gdn_status gdn_workspace_size(const gdn_problem* problem, int32_t pass, size_t* bytes);

/* Forward pass of the chunked gated delta rule.
 *   in : q, k, v, g, beta; S0 (NULL = zero initial state)
 *   out: o; S_final (NULL = not wanted)
 * Chunk algebra per (sequence, head), chunk of n <= 64 tokens, state S_c before it:
 *   gamma = cumsum(g) within the chunk; D_ij = exp(gamma_i - gamma_j) (j <= i)
 *   A = strict_lower(diag(beta) (K K^T) o D); T = (I + A)^-1 (unit lower triangular)
 *   E = T diag(beta) (V - diag(exp(gamma)) K S_c)      (the errors e_t of the chunk)
 *   O = scale (diag(exp(gamma)) Q S_c + lower_incl(Q K^T o D) E)
 *   S_{c+1} = exp(gamma_n) S_c + (diag(exp(gamma_n - gamma)) K)^T E
 * num_segments = G > 1 splits every sequence of nch chunks into G runs of whole
 * chunks (segment s covers chunks [s L, min((s + 1) L, nch)), L = ceil(nch / G))
 * that run in parallel: each segment's state map S -> M S + b is taken by the
 * same chunk pass (b from a zero start, M from the identity with V = 0), the
 * start states are composed in fp32 in segment order, and the segments are run
 * again from them with their outputs (cuLA issue #126 page, "Summary" and
 * "Hypothesis": segment affine transforms and carries).  G = 2 gives results
 * bit-identical to G = 1; G > 2 agrees to the bf16 rounding of M's operands.
 * Workspace: gdn_workspace_size(..., GDN_PASS_CHUNK_FWD, ...): per chunk and
 * head, T diag(beta) (its 16x16 blocks on and below the diagonal), the causal
 * score and the chunk's decays, plus for G > 1 fp32 buffers of
 * 2 G N H Dk Dv + G N H Dk Dk floats. */
gdn_status gdn_chunk_fwd(const gdn_problem* problem, const void* q, const void* k,
                         const void* v, const float* g, const float* beta, const float* S0,
                         void* o, float* S_final, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Size of the device array that gdn_chunk_fwd_noalloc uses as its workspace
 * (64 MiB: the bf16 forward of 4 x 4096 tokens x 8 heads at Dk = Dv = 128 needs
 * about 30 MiB). */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* gdn_chunk_fwd without a caller-provided workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops or
 * harnesses that forbid allocation).  Same arguments, results and kernels as
 * gdn_chunk_fwd; the workspace is a file-scope device array of
 * GDN_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on
 * until the process ends.  The call allocates nothing: the array's device
 * address is looked up once per device (on the first call with that device
 * current; the current device must be the one `stream` belongs to).
 *   Errors: as gdn_chunk_fwd, plus GDN_ERR_SCRATCH (before any launch) when
 *   gdn_workspace_size(problem, GDN_PASS_CHUNK_FWD) exceeds the array, and
 *   GDN_ERR_HIP if the address lookup fails.
 *   Concurrency: every call on one device shares that device's array, which
 *   keeps the last call's contents (nothing in it has to start at zero).  Calls
 *   whose executions overlap on one device -- different streams, or different
 *   host threads -- race on the array and give undefined results; serialise
 *   them (one stream, or events). */
gdn_status gdn_chunk_fwd_noalloc(const gdn_problem* problem, const void* q, const void* k,
                                 const void* v, const float* g, const float* beta, const float* S0,
                                 void* o, float* S_final, void* stream);

/* Backward pass of the chunked gated delta rule: gradients of
 *   L = <o, dO> + <S_final, dS_final>
 * with respect to q, k, v, g, beta and S0 (the six gradients of the Day-1 page's
 * "Results" tables plus the initial-state gradient).
 *   in : q, k, v, g, beta, S0 (NULL = zero), dO, dS_final (NULL = zero)
 *   out: dq, dk, dv (io dtype), dg, dbeta (fp32), dS0 (fp32; NULL = not wanted)
 * num_segments must be 1.  Workspace: GDN_PASS_CHUNK_BWD (T, T diag(beta), the
 * decays and the causal score P of every chunk, and the state before and its
 * gradient after every chunk, held in the products' operand type: bf16 for bf16
 * io, fp32 for fp32 io, the type in which the gradient products consume them). */
gdn_status gdn_chunk_bwd(const gdn_problem* problem, const void* q, const void* k,
                         const void* v, const float* g, const float* beta, const float* S0,
                         const void* dO, const float* dS_final, void* dq, void* dk, void* dv,
                         float* dg, float* dbeta, float* dS0, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Training with retained states: the forward keeps what the backward needs, so
 * the backward does not run the forward's state pass again (the fla issue #1550
 * page, "Proposed scope", asks for retained or recomputed states as a measured
 * choice; gdn_chunk_bwd is the recomputing one).
 *
 * gdn_chunk_fwd_save computes exactly what gdn_chunk_fwd computes (o, S_final;
 * the same arithmetic, so bit-identical results) and also fills `saved` with
 * T, T diag(beta), the decays and the causal score P of every chunk and the state
 * before every chunk (in the operand type, as for gdn_chunk_bwd).  gdn_chunk_bwd_saved then runs only the reverse
 * passes of gdn_chunk_bwd and gives bit-identical gradients, provided q, k, v, g,
 * beta, S0 and the problem are the same as in the gdn_chunk_fwd_save call and
 * `saved` was not modified in between (neither is checked: other contents give
 * undefined gradients, not an error).  gdn_chunk_bwd_saved writes the state
 * gradients into `saved` as well; `saved` may be reused for the next step.
 *   saved: caller-allocated device buffer of gdn_workspace_size(problem,
 *          GDN_PASS_CHUNK_SAVED) bytes (the backward workspace plus P in the
 *          forward's operand order), 16-byte aligned.
 *   Supported and errors: as gdn_chunk_bwd (num_segments 1, precision IO).
 *   S0 is not an argument of gdn_chunk_bwd_saved (the saved states carry it);
 *   dS0 is still produced. */
gdn_status gdn_chunk_fwd_save(const gdn_problem* problem, const void* q, const void* k,
                              const void* v, const float* g, const float* beta, const float* S0,
                              void* o, float* S_final, void* saved, size_t saved_bytes,
                              void* stream);
gdn_status gdn_chunk_bwd_saved(const gdn_problem* problem, const void* q, const void* k,
                               const void* v, const float* g, const float* beta, const void* dO,
                               const float* dS_final, void* dq, void* dk, void* dv, float* dg,
                               float* dbeta, float* dS0, void* saved, size_t saved_bytes,
                               void* stream);

/* Token-by-token recurrence in IEEE fp32 on the GPU: the full-length second
 * reference (not the fast path).  Forward always (o, S_final as gdn_chunk_fwd).
 * If dO is non-NULL it also runs the token-level reverse mode and writes dq, dk,
 * dv, dg, dbeta (all required then) and dS0 (optional), like gdn_chunk_bwd.
 * num_segments is ignored.  Workspace: GDN_PASS_RECURRENT_FWD when dO == NULL,
 * else GDN_PASS_RECURRENT_BWD. */
gdn_status gdn_recurrent_ref(const gdn_problem* problem, const void* q, const void* k,
                             const void* v, const float* g, const float* beta,
                             const float* S0, void* o, float* S_final, const void* dO,
                             const float* dS_final, void* dq, void* dk, void* dv, float* dg,
                             float* dbeta, float* dS0, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Chunked forward pass with one log-decay per key channel: the gate layout of
 * the cuLA issue #126 page ("Minimal public reproduction", where g has the shape
 * of q and is handed to the KDA kernels).  Per token, with a = exp(g_t) a vector
 * of Dk factors:  S <- diag(a) S,  e = beta (v - S^T k),  S <- S + k e^T,
 * o = scale S^T q  (the update of "Research Sprint Day 1", "The GDN update",
 * with a diagonal forget factor; with equal factors on every channel it is
 * gdn_chunk_fwd's recurrence).
 *   in : q, k [B,T,H,Dk] and v [B,T,H,Dv] (io dtype); g [B,T,H,Dk] fp32, finite
 *        and <= 0; beta [B,T,H] fp32; S0 [N,H,Dk,Dv] fp32 or NULL (zero)
 *   out: o [B,T,H,Dv] (io dtype), S_final [N,H,Dk,Dv] fp32 or NULL
 * Packed sequences through cu_seqlens as for gdn_chunk_fwd.  Dk 64 or 128 and
 * Dv a multiple of 16 up to 256, for both io dtypes.  num_segments in {1, 2, 4,
 * 8, 16}: the segment split of gdn_chunk_fwd (segment maps S -> M S + b, M a
 * Dk x Dk matrix, composed in fp32; G = 2 and the first two segments are
 * bit-identical to G = 1) -- the intra-card split whose error the cuLA issue
 * #126 page measures ("Summary").
 * Precision: decays, A, the inverse and the state are fp32; the products take
 * bf16 operands with fp32 accumulation for bf16 io and are IEEE fp32 for fp32 io.
 * Workspace: gdn_workspace_size(..., GDN_PASS_KDA_FWD, ...): one record per chunk
 * and head (T diag(beta), the causal score, K and Q scaled by the decays, the
 * decayed keys of the state update, in the io element type; the chunk's decay),
 * then for G > 1 fp32 buffers of 2 G N H Dk Dv + G N H Dk Dk floats.  Errors as gdn_chunk_fwd: every check
 * runs before the first launch. */
gdn_status gdn_kda_chunk_fwd(const gdn_problem* problem, const void* q, const void* k,
                             const void* v, const float* g, const float* beta, const float* S0,
                             void* o, float* S_final, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Reverse mode of gdn_kda_chunk_fwd: the gradients of
 *   L = <o, dO> + <S_final, dS_final>
 * with respect to q, k, v, the per-channel log-decays g, beta and S0, for the
 * recurrence of gdn_kda_chunk_fwd (per token, a = exp(g_t) of length Dk:
 * S <- diag(a) S, e = beta (v - S^T k), S <- S + k e^T, o = scale S^T q; the
 * update of "Research Sprint Day 1", "The GDN update", with the diagonal forget
 * factor of the cuLA issue #126 page's gate layout).
 *   in : q, k, v, g, beta, S0 (NULL = zero) as gdn_kda_chunk_fwd; dO [B,T,H,Dv]
 *        (io dtype); dS_final [N,H,Dk,Dv] fp32 or NULL (zero)
 *   out: dq, dk [B,T,H,Dk] and dv [B,T,H,Dv] (io dtype); dg [B,T,H,Dk] fp32 (one
 *        gradient per key channel); dbeta [B,T,H] fp32; dS0 [N,H,Dk,Dv] fp32
 *        (NULL = not wanted)
 * The forward's chunk preparation and state pass run again (no o is written);
 * then a reverse pass over the chunks forms the state gradient after every
 * chunk, and one workgroup per chunk forms its gradients.  Packed sequences as
 * for gdn_kda_chunk_fwd; Dk 64 or 128, Dv a multiple of 16 up to 256, both io
 * dtypes; num_segments must be 1 and precision GDN_PRECISION_IO.
 * Precision: decays, the inverse, the state and its gradient are fp32; the
 * products take bf16 operands with fp32 accumulation for bf16 io (the records,
 * the per-chunk states and state gradients, and the intermediate tiles rounded to
 * bf16) and are IEEE fp32 for fp32 io; the pair sums through the per-channel
 * decays are fp32 for both.
 * Workspace: gdn_workspace_size(..., GDN_PASS_KDA_BWD, ...): the forward's records,
 * then per chunk and head 12288 floats (T, Ab, P in fp32) and the state before and
 * its gradient after the chunk, Dk Dv values each in the io element type.  Errors
 * as gdn_kda_chunk_fwd. */
gdn_status gdn_kda_chunk_bwd(const gdn_problem* problem, const void* q, const void* k,
                             const void* v, const float* g, const float* beta, const float* S0,
                             const void* dO, const float* dS_final, void* dq, void* dk, void* dv,
                             float* dg, float* dbeta, float* dS0, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Training with retained states for the per-channel decay, as gdn_chunk_fwd_save /
 * gdn_chunk_bwd_saved for the scalar gate (the fla issue #1550 page, "Proposed
 * scope": retained or recomputed states).  gdn_kda_chunk_fwd_save computes exactly
 * what gdn_kda_chunk_fwd computes with num_segments = 1 (o, S_final; bit-identical)
 * and also fills `saved` with the chunk records, fp32 T, Ab and P, and the state
 * before every chunk; gdn_kda_chunk_bwd_saved then runs only the reverse passes of
 * gdn_kda_chunk_bwd and gives bit-identical gradients, provided q, k, v, g, beta, S0
 * and the problem are those of the save call and `saved` was not modified in
 * between (neither is checked: other contents give undefined gradients, not an
 * error).  It writes the state gradients into `saved` as well.
 *   saved: caller-allocated device buffer of gdn_workspace_size(problem,
 *          GDN_PASS_KDA_SAVED) bytes (the gdn_kda_chunk_bwd workspace), 16-byte
 *          aligned.
 *   Supported and errors: as gdn_kda_chunk_bwd.  S0 is not an argument of
 *   gdn_kda_chunk_bwd_saved (the saved states carry it); dS0 is still produced. */
gdn_status gdn_kda_chunk_fwd_save(const gdn_problem* problem, const void* q, const void* k,
                                  const void* v, const float* g, const float* beta, const float* S0,
                                  void* o, float* S_final, void* saved, size_t saved_bytes,
                                  void* stream);
gdn_status gdn_kda_chunk_bwd_saved(const gdn_problem* problem, const void* q, const void* k,
                                   const void* v, const float* g, const float* beta, const void* dO,
                                   const float* dS_final, void* dq, void* dk, void* dv, float* dg,
                                   float* dbeta, float* dS0, void* saved, size_t saved_bytes,
                                   void* stream);

/* Gate forms of gdn_prologue. */
typedef enum {
  GDN_GATE_GDN = 0,         /* g = -exp(A_log[h]) * softplus(a + dt_bias[h])            */
  GDN_GATE_BOUNDED5 = 1,    /* g = -5 * sigmoid(a), in (-5, 0)                          */
  GDN_GATE_GDN_CHANNEL = 2  /* g[..., c] = -exp(A_log[h]) * softplus(a[..., c] + dt_bias[h, c]) */
} gdn_gate_kind;

/* Fused input prologue: the elementwise step that produces the operator's inputs
 * from the raw projections, in one pass over HBM.
 *   q_out = q / max(||q||_2, 1e-30), k_out = k / max(||k||_2, 1e-30): norms over
 *           the last dimension in fp32 from the io-dtype inputs, then rounded to
 *           the io dtype (round to nearest even).  The fla issue #1550 page
 *           ("Proposed scope") asks for exactly this order: normalise in FP32,
 *           then cast.
 *   beta  = sigmoid(b), or 2 sigmoid(b) when allow_neg_eigval != 0 (the range
 *           (0, 2) of the Day-2 page, "Building some intuition", gates).
 *   g     = -exp(A_log[h]) softplus(a + dt_bias[h])   (GDN_GATE_GDN: the gate
 *           formula of the Day-2 page, "Building some intuition", steps 4-5), or
 *           -5 sigmoid(a)                              (GDN_GATE_BOUNDED5: the
 *           bounded gates of the fla issue #1550 workload), or the first form
 *           channel by channel, one log-decay per key channel for
 *           gdn_kda_chunk_fwd (GDN_GATE_GDN_CHANNEL: the gate layout of the cuLA
 *           issue #126 page, "Minimal public reproduction", dt_bias per head and
 *           channel).
 * Shapes: q, k, q_out, k_out [B, T, H, Dk] io dtype; b, beta [B, T, H] fp32; a, g
 * [B, T, H] fp32, or [B, T, H, Dk] for GDN_GATE_GDN_CHANNEL; A_log [H] fp32 and
 * dt_bias [H] fp32, or [H, Dk] for GDN_GATE_GDN_CHANNEL (both required for the
 * two GDN forms, ignored for GDN_GATE_BOUNDED5).
 * `problem` is the problem of the chunked call the outputs feed (only B, T, H,
 * Dk and io_dtype are used; it is validated as for gdn_recurrent_ref).  Outputs
 * must not overlap inputs (GDN_ERR_ALIAS).  No workspace.  In fp32 the results
 * are the correctly computed fp32 expressions up to a few units of the last
 * place (the exponentials and the division). */
gdn_status gdn_prologue(const gdn_problem* problem, const void* q, const void* k, const float* a,
                        const float* b, const float* A_log, const float* dt_bias, int32_t gate_kind,
                        int32_t allow_neg_eigval, void* q_out, void* k_out, float* g, float* beta,
                        void* stream);

/* Output epilogue: the gated, normalised output the operator's result feeds,
 * in one pass over HBM ("Research Sprint Day 2", "Building some intuition",
 * step 7: normalise per head, then gate):
 *   y = o / sqrt(mean_j(o_j^2) + eps) * weight * silu(z),  silu(z) = z sigmoid(z)
 * per (token, head) over the Dv values, in fp32, rounded once to the io dtype.
 * Shapes: o, z, y [B, T, H, Dv] io dtype; weight [Dv] fp32, 16-byte aligned (NULL =
 * all ones).
 * eps >= 0 is documented, not checked.  `problem` is that of the chunked call
 * that produced o (B, T, H, Dv and io_dtype are used; validated as for
 * gdn_recurrent_ref); Dv must be a power of two (16 .. 256), else
 * GDN_ERR_UNSUPPORTED.  y must not overlap o or z (GDN_ERR_ALIAS).  No workspace. */
gdn_status gdn_epilogue(const gdn_problem* problem, const void* o, const void* z, const float* weight,
                        float eps, void* y, void* stream);

/* Measurement helper, not part of the operator: copies `bytes` bytes of device
 * memory from src to dst (16-byte vectors, non-temporal, grid-strided), the copy
 * that calibrates the HBM roofline the chunked kernels are measured against
 * ("Research Sprint Day 2 - Rooflines", section "Rooflines": the bandwidth of a
 * large copy, bytes read plus bytes written).  dst, src and bytes must be
 * multiples of 16 (GDN_ERR_ALIGN), the ranges must not overlap (GDN_ERR_ALIAS);
 * asynchronous on `stream`. */
gdn_status gdn_device_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
