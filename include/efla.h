/*
 * efla.h - C ABI of the MI355X (gfx950) Exact Flow Linear Attention library.
 *
 * The operator ("Exact Flow Linear Attention: Exact Solution from
 * Continuous-Time Dynamics", gist.science Technical Summary, Methodology 3):
 * for each (batch b, head h) independently and t = 0 .. L-1,
 *
 *     lambda_t = |k_t|^2,   alpha_t = (1 - exp(-beta_t lambda_t)) / lambda_t
 *                                     (= beta_t in the limit lambda_t -> 0)
 *     S_t = (I - alpha_t k_t k_t^T) S_{t-1} + alpha_t k_t v_t^T
 *     o_t = S_t^T q_t                       (the state after the update)
 *
 * S_t is d_k x d_v.  The update keeps the delta rule's rank-1 form, which is
 * what lets the chunkwise (WY/UT) evaluation used here reproduce the token
 * recurrence (Methodology 3; the pages name the scheme without formulas).
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are HIP device pointers owned by the caller.  Tensors are
 *    row-major and contiguous in the layouts given below; every pointer must be
 *    16-byte aligned.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Outputs are valid once the caller has synchronised the stream.
 *  - Arguments are validated before any HIP call.  A call that returns an
 *    error status has launched nothing.  The library never prints, never
 *    aborts and never allocates device memory.
 *  - Distinct calls are thread-safe when they use distinct streams and
 *    buffers.
 *  - Supported shapes: d_k, d_v in {16, 32, 64, 128}; chunk in {16, 32, 64}.
 *    Other values return EFLA_ERR_UNSUPPORTED.
 *  - Any L >= 0 is accepted.  A last partial chunk is evaluated exactly:
 *    missing tokens act as alpha = 0, which is the identity update.
 *  - beta may hold any finite value; no clamp is applied.
 */
#ifndef EFLA_H
#define EFLA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v, o (and of the W, U, A stage outputs).  The state,
 * beta, alpha and lambda are always fp32.  bf16 inputs are multiplied on bf16
 * MFMA with fp32 accumulation; fp32 inputs on fp32 MFMA. */
typedef enum { EFLA_F32 = 0, EFLA_BF16 = 1 } efla_dtype_t;

typedef enum {
    EFLA_OK = 0,
    EFLA_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, negative size, bad enum */
    EFLA_ERR_UNSUPPORTED = 2,  /* d_k, d_v or chunk outside the supported set      */
    EFLA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required       */
    EFLA_ERR_HIP = 4           /* a HIP launch reported an error                   */
} efla_status_t;

/* Evaluation strategy of efla_forward_ex.  AUTO takes FUSED for bf16 inputs
 * unless the fused kernel would run at most 32 workgroups (one per sequence
 * and 32 state columns) and the sequences are long enough to split, then
 * SEGMENTED; for fp32, SEGMENTED when the sequences are too few to fill the
 * GPU and long enough to split, else STAGED. */
typedef enum {
    EFLA_PATH_AUTO = 0,    /* the fastest path available for the shape         */
    EFLA_PATH_STAGED = 1,  /* UT transform (with the coefficients) -> state
                              scan: the stages below, with W, U and A in the
                              workspace                                      */
    EFLA_PATH_FUSED = 2,   /* one kernel; no intermediate HBM traffic           */
    EFLA_PATH_SEGMENTED = 3 /* staged, with the state scan split over L into
                               segments: each segment's affine map S -> P S + R
                               is formed in parallel, the maps are composed into
                               every segment's entry state, and the segments are
                               replayed in parallel (for few, long sequences) */
} efla_path_t;

/* Coefficient of the update.
 *  EFLA_EXACT: alpha = (1 - exp(-beta lambda)) / lambda, the exact flow
 *              (Methodology 2-3); what efla_forward, efla_forward_ex,
 *              efla_decode_step and efla_coefficients compute.
 *  EFLA_EULER: alpha = beta, the explicit Euler step of the same ODE -- the
 *              delta rule the pages compare the exact flow against (Problem
 *              Statement).  Same kernels, layouts and rules; only alpha
 *              differs.
 * Any other value returns EFLA_ERR_INVALID_ARG. */
typedef enum { EFLA_EXACT = 0, EFLA_EULER = 1 } efla_update_t;

/* Launch shape of the chunked kernels, for callers that tune them.  Each
 * field chosen as 0 takes the library's built-in choice; a NULL pointer means
 * all zero.  The values pick other compiled instances of the same kernels
 * (how many 16-column tiles of the state one workgroup owns); the arithmetic
 * of every column, and so the result, does not depend on them.
 *   fused_scan_waves  fused forward: 1 or 2 scan waves per workgroup
 *                     (16- or 32-column state tiles)
 *   scan_waves        staged and segmented state scans: 1, 2, 4 or 8 waves per
 *                     workgroup (8 only for fp32 inputs at d_k = d_v = 128, the
 *                     built-in choice of the segmented passes there; elsewhere
 *                     it acts as 4)
 *   bwd_scan_waves    the backward's two state scans: 1, 2 or 4
 * Any other value returns EFLA_ERR_INVALID_ARG.  The library reads no
 * environment variable and keeps no setting between calls. */
typedef struct {
    int fused_scan_waves;
    int scan_waves;
    int bwd_scan_waves;
} efla_launch_config_t;

/* The path EFLA_PATH_AUTO takes for this shape (EFLA_PATH_AUTO itself for an
 * invalid shape). */
efla_path_t efla_forward_path(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype_t dt);

/* Human-readable name of a status code (static storage, never NULL). */
const char *efla_status_string(efla_status_t s);

/* Bytes of device workspace efla_forward / efla_forward_ex(path) needs for
 * this shape (0 when the path needs none).  Returns 0 for invalid shapes. */
size_t efla_forward_workspace_size(int B, int H, int L, int d_k, int d_v, int chunk,
                                   efla_dtype_t dt);
size_t efla_forward_workspace_size_ex(int B, int H, int L, int d_k, int d_v, int chunk,
                                      efla_dtype_t dt, efla_path_t path);

/*
 * Chunked forward over whole sequences (Methodology 3).
 *   q, k  [B,H,L,d_k]  dtype dt           v  [B,H,L,d_v]  dtype dt
 *   beta  [B,H,L]      fp32               per token and head
 *   S0    [B,H,d_k,d_v] fp32 or NULL      NULL means the zero initial state
 *   o     [B,H,L,d_v]  dtype dt           output, o_t = S_t^T q_t
 *   S_L   [B,H,d_k,d_v] fp32              output, state after token L-1;
 *                                          may alias S0 (exactly the same
 *                                          pointer), no other aliasing
 *   workspace: device buffer of at least efla_forward_workspace_size() bytes,
 *   256-byte aligned, owned by the caller; it may be NULL when that size is 0.
 * With L = 0, S_L receives S0 (or zeros) and o is untouched.
 */
efla_status_t efla_forward(const void *q, const void *k, const void *v, const float *beta,
                           const float *S0, void *o, float *S_L,
                           int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype_t dt,
                           void *workspace, size_t workspace_bytes, void *stream);

/* efla_forward with an explicit evaluation path; results agree with the
 * token recurrence to within fp32/bf16 rounding whichever path runs. */
efla_status_t efla_forward_ex(const void *q, const void *k, const void *v, const float *beta,
                              const float *S0, void *o, float *S_L,
                              int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype_t dt,
                              void *workspace, size_t workspace_bytes, efla_path_t path,
                              void *stream);

/*
 * Chunked forward over N packed sequences of varying length (Methodology 3;
 * each sequence is an independent recurrence, so its chunks restart at its
 * first token).
 *   q, k [H,T,d_k], v [H,T,d_v] dtype dt; beta [H,T] fp32: for each head the N
 *        sequences back to back along the T-token axis, sequence n at tokens
 *        [cu_seqlens[n], cu_seqlens[n+1])
 *   cu_seqlens  device int32 [N+1], non-decreasing, cu_seqlens[0] = 0,
 *        cu_seqlens[N] <= T.  Offsets outside [0, T] are clamped into it (the
 *        sequence shrinks; no access leaves the tensors).
 *   S0   [N,H,d_k,d_v] fp32 or NULL (zero state); S_L [N,H,d_k,d_v] fp32 out,
 *        may alias S0 exactly
 *   o    [H,T,d_v] dtype dt; tokens outside every sequence are left untouched
 * Runs the fused kernel and needs no workspace: dt must be EFLA_BF16, else
 * EFLA_ERR_UNSUPPORTED (efla_forward_varlen_ex takes fp32 and the other
 * paths).
 */
efla_status_t efla_forward_varlen(const void *q, const void *k, const void *v, const float *beta,
                                  const int *cu_seqlens, const float *S0, void *o, float *S_L,
                                  int N, int H, int T, int d_k, int d_v, int chunk,
                                  efla_dtype_t dt, efla_update_t update, void *stream);

/* Workspace bytes efla_forward_varlen_ex needs on `path` for these sizes (0
 * for the fused path, or for invalid arguments).  It depends on N, H, T and
 * the shape only, not on the offsets. */
size_t efla_forward_varlen_workspace_size(int N, int H, int T, int d_k, int d_v, int chunk,
                                          efla_dtype_t dt, efla_path_t path);

/*
 * efla_forward_varlen on any evaluation path, for fp32 and bf16 inputs
 * (Methodology 3; each packed sequence is its own recurrence).  Arguments,
 * layouts, clamping of offsets and results as for efla_forward_varlen, plus:
 *   path  EFLA_PATH_FUSED (bf16 only, no workspace), EFLA_PATH_STAGED (UT
 *         transform, state scan; one scan per (sequence, head)),
 *         EFLA_PATH_SEGMENTED (the scan split into segment maps, their
 *         composition and a replay: for few long sequences), or
 *         EFLA_PATH_AUTO (bf16 as for efla_forward_ex; fp32: segmented
 *         when N * H * ceil(d_v / 64) < 256 and a sequence as long as the
 *         whole token axis would be split, else staged; the segment plan is
 *         made for such a sequence)
 *   workspace  device buffer of efla_forward_varlen_workspace_size(...)
 *         bytes, 256-byte aligned, owned by the caller (NULL allowed when
 *         that size is 0 or T = 0); too small: EFLA_ERR_WORKSPACE
 * Tokens outside every sequence are not read on the staged and segmented
 * paths.
 */
efla_status_t efla_forward_varlen_ex(const void *q, const void *k, const void *v,
                                     const float *beta, const int *cu_seqlens, const float *S0,
                                     void *o, float *S_L, int N, int H, int T, int d_k, int d_v,
                                     int chunk, efla_dtype_t dt, efla_update_t update,
                                     efla_path_t path, void *workspace, size_t workspace_bytes,
                                     void *stream);

/* efla_forward_ex with an explicit update (EFLA_EXACT or EFLA_EULER). */
efla_status_t efla_forward_update(const void *q, const void *k, const void *v, const float *beta,
                                  const float *S0, void *o, float *S_L,
                                  int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype_t dt,
                                  void *workspace, size_t workspace_bytes, efla_path_t path,
                                  efla_update_t update, void *stream);

/* efla_forward_update with an explicit launch configuration (NULL = the
 * built-in one).  Same results as efla_forward_update. */
efla_status_t efla_forward_config(const void *q, const void *k, const void *v, const float *beta,
                                  const float *S0, void *o, float *S_L,
                                  int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype_t dt,
                                  void *workspace, size_t workspace_bytes, efla_path_t path,
                                  efla_update_t update, const efla_launch_config_t *config,
                                  void *stream);

/*
 * Allocation-free chunked forward, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): efla_forward_update without a workspace argument.  The
 * fused path needs no workspace; the staged and segmented paths keep their
 * intermediates (W, U, A and the segment maps) in a device array of
 * EFLA_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs
 * on until the process ends.  A shape whose workspace on the path taken
 * (efla_forward_workspace_size_ex) exceeds that size returns
 * EFLA_ERR_WORKSPACE with nothing launched; with EFLA_PATH_AUTO, bf16 inputs
 * then take the fused kernel instead (which needs none).  This entry calls no hipMalloc,
 * hipFree or allocating routine.  Every call on one device shares the array
 * and relies on nothing it held before (each call writes every intermediate
 * it reads): calls that overlap in time on one device -- on different streams,
 * or from host threads without ordering -- race, and the caller must
 * serialize them.  The first call on a device looks up the array's device
 * address (hipGetSymbolAddress, with that device current) and keeps it.
 * Arguments, layouts and results as for efla_forward_update.
 */
#define EFLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
efla_status_t efla_forward_noalloc(const void *q, const void *k, const void *v, const float *beta,
                                   const float *S0, void *o, float *S_L,
                                   int B, int H, int L, int d_k, int d_v, int chunk,
                                   efla_dtype_t dt, efla_path_t path, efla_update_t update,
                                   void *stream);

/*
 * Single-token decode step (the recurrent form of the same update) for N
 * sequences x H heads, in place:
 *   q, k [N,H,d_k]  v [N,H,d_v]  dtype dt;  beta [N,H] fp32
 *   S    [N,H,d_k,d_v] fp32, read and overwritten with S_new
 *   o    [N,H,d_v]  dtype dt, o = S_new^T q
 * Each (n,h) state is read completely before any of it is written.
 */
efla_status_t efla_decode_step(const void *q, const void *k, const void *v, const float *beta,
                               float *S, void *o, int N, int H, int d_k, int d_v,
                               efla_dtype_t dt, void *stream);

/* efla_decode_step with an explicit update (EFLA_EXACT or EFLA_EULER). */
efla_status_t efla_decode_step_update(const void *q, const void *k, const void *v,
                                      const float *beta, float *S, void *o, int N, int H,
                                      int d_k, int d_v, efla_dtype_t dt, efla_update_t update,
                                      void *stream);

/*
 * Single-token decode step for a ragged serving batch whose states live in a
 * pool (Methodology 3, the recurrent form): token n of the batch belongs to
 * the sequence whose state is pool entry slots[n], and updates it in place.
 * No gather or scatter of states: each token's workgroup reads and writes its
 * pool entry directly.
 *   q, k [N,H,d_k], v [N,H,d_v] dtype dt; beta [N,H] fp32; o [N,H,d_v] dtype dt
 *   slots   device int32 [N]; entries must be distinct and in [0, P)
 *   S_pool  [P,H,d_k,d_v] fp32: entries slots[n] read and overwritten (each
 *           read completely before any of it is written), all others untouched
 *   err     device int32 or NULL.  A slot outside [0, P) or named by more than
 *           one token is rejected on the device: the tokens naming it leave
 *           the pool untouched, get o = NaN, and OR 2 (out of range) or 1
 *           (repeated) into *err.  The library never clears *err.
 * N = 0 is valid and launches nothing.  Other arguments as for
 * efla_decode_step_update.
 */
efla_status_t efla_decode_step_indexed(const void *q, const void *k, const void *v,
                                       const float *beta, const int *slots, float *S_pool,
                                       void *o, int *err, int N, int H, int P, int d_k, int d_v,
                                       efla_dtype_t dt, efla_update_t update, void *stream);

/*
 * Per-token coefficients (Methodology 2-3): the first stage of the chunked
 * form, exported on its own.  (The forward entry points form them inside
 * their UT transform or fused kernel, from the same formula.)
 *   k [n_tokens, d_k] dtype dt; beta [n_tokens] fp32
 *   alpha [n_tokens] fp32 out; lambda [n_tokens] fp32 out, or NULL to skip.
 * lambda_t = |k_t|^2 accumulated in fp32 from the stored k; with
 * x = beta_t lambda_t, alpha_t = beta_t phi(x), phi(x) = (1 - e^{-x}) / x from
 * its Taylor series for |x| < 1/2 (so alpha_t = beta_t at lambda_t = 0), and
 * (1 - e^{-x}) / lambda_t otherwise.
 */
efla_status_t efla_coefficients(const void *k, const float *beta, float *alpha, float *lambda,
                                long n_tokens, int d_k, efla_dtype_t dt, void *stream);

/* efla_coefficients with an explicit update: EFLA_EULER writes alpha = beta
 * (lambda is still |k|^2). */
efla_status_t efla_coefficients_update(const void *k, const float *beta, float *alpha,
                                       float *lambda, long n_tokens, int d_k, efla_dtype_t dt,
                                       efla_update_t update, void *stream);

/*
 * Stage 2: per-chunk UT transform.  For every chunk of `chunk` consecutive
 * tokens of every (b,h) (last chunk possibly partial), with K, V the chunk's
 * keys and values and a = alpha:
 *   T = (I + strictly_lower(diag(a) K K^T))^{-1} diag(a)   (fp32, forward
 *        substitution on 16x16 diagonal blocks, block substitution off them)
 *   W = T K  -> w [B,H,L,d_k] dtype dt
 *   U = T V  -> u [B,H,L,d_v] dtype dt
 *   A = tril(Q K^T), diagonal included -> a_qk [B,H,ceil(L/chunk),chunk,chunk]
 *       dtype dt (rows/columns past L are zero)
 *   q, k [B,H,L,d_k], v [B,H,L,d_v] dtype dt; alpha [B,H,L] fp32.
 */
efla_status_t efla_ut_transform(const void *q, const void *k, const void *v, const float *alpha,
                                void *w, void *u, void *a_qk,
                                int B, int H, int L, int d_k, int d_v, int chunk,
                                efla_dtype_t dt, void *stream);

/*
 * Stage 3: inter-chunk state scan.  Per (b,h) the fp32 state S (from S0, or
 * zero) stays on chip; for each chunk in order
 *   E = U - W S;   O = Q S + A E;   S <- S + K^T E
 * with W, U, A from stage 2.  Writes o [B,H,L,d_v] (dtype dt) and S_L.
 * S_L may alias S0 exactly.
 */
efla_status_t efla_chunk_scan(const void *q, const void *k, const void *w, const void *u,
                              const void *a_qk, const float *S0, void *o, float *S_L,
                              int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype_t dt,
                              void *stream);

/*
 * Backward pass of the chunked forward: the gradients of a scalar loss with
 * respect to every input, given its gradients with respect to the outputs.
 * The pages train models with the exact-flow layer (Experiments) but print
 * no backward; this is the adjoint of the forward defined above, evaluated
 * chunkwise.
 *   q, k, v, beta, S0  the forward's inputs, as for efla_forward (S0 NULL =
 *                      zero initial state)
 *   d_o   [B,H,L,d_v]   dtype dt   dLoss/do
 *   dS_L  [B,H,d_k,d_v] fp32       dLoss/dS_L, or NULL for zero
 *   dq, dk [B,H,L,d_k], dv [B,H,L,d_v]  dtype dt, outputs
 *   dbeta [B,H,L] fp32, output
 *   dS0   [B,H,d_k,d_v] fp32 output (dLoss/dS0), or NULL if not wanted
 *   update  EFLA_EXACT or EFLA_EULER: the update the forward used
 *   workspace: at least efla_backward_workspace_size() bytes, 256-byte
 *   aligned, owned by the caller (NULL allowed when that size is 0).
 * dbeta uses d alpha / d beta = exp(-beta lambda) and dk includes the path
 * through lambda = |k|^2 (d alpha / d lambda); for EFLA_EULER these are 1
 * and 0.  The forward is recomputed inside (coefficients, UT transform and
 * the state scan, which stores every chunk's entry state), then a reverse
 * scan carries dLoss/dS from the last chunk to the first and a per-chunk
 * kernel forms dq, dk, dv and dbeta.  As in the forward, bf16 inputs are
 * multiplied on bf16 MFMA and fp32 inputs on fp32 MFMA, accumulating in fp32;
 * the triangular solves stay fp32.  No output may alias an input or another
 * output.
 * With L = 0 only dS0 = dS_L (or zeros) is written.
 */
size_t efla_backward_workspace_size(int B, int H, int L, int d_k, int d_v, int chunk,
                                    efla_dtype_t dt);

efla_status_t efla_backward(const void *q, const void *k, const void *v, const float *beta,
                            const float *S0, const void *d_o, const float *dS_L,
                            void *dq, void *dk, void *dv, float *dbeta, float *dS0,
                            int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype_t dt,
                            efla_update_t update, void *workspace, size_t workspace_bytes,
                            void *stream);

/* efla_backward with an explicit launch configuration (NULL = the built-in
 * one).  Same results as efla_backward. */
efla_status_t efla_backward_config(const void *q, const void *k, const void *v, const float *beta,
                                   const float *S0, const void *d_o, const float *dS_L,
                                   void *dq, void *dk, void *dv, float *dbeta, float *dS0,
                                   int B, int H, int L, int d_k, int d_v, int chunk,
                                   efla_dtype_t dt, efla_update_t update,
                                   const efla_launch_config_t *config, void *workspace,
                                   size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* EFLA_H */
