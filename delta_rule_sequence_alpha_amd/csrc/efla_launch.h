// Internal host-side launchers of the EFLA kernels (C++ linkage, not exported).
#pragma once

#include <hip/hip_runtime.h>

// Every (d_k, d_v, chunk) the chunked kernels are instantiated for:
// d_k, d_v in {16, 32, 64, 128} x chunk in {16, 32, 64}.
#define EFLA_SHAPES_FOR_C(X, CC)                                                                 \
    X(16, 16, CC) X(16, 32, CC) X(16, 64, CC) X(16, 128, CC)                                     \
    X(32, 16, CC) X(32, 32, CC) X(32, 64, CC) X(32, 128, CC)                                     \
    X(64, 16, CC) X(64, 32, CC) X(64, 64, CC) X(64, 128, CC)                                     \
    X(128, 16, CC) X(128, 32, CC) X(128, 64, CC) X(128, 128, CC)
#define EFLA_SHAPE_CASES(X) EFLA_SHAPES_FOR_C(X, 16) EFLA_SHAPES_FOR_C(X, 32) EFLA_SHAPES_FOR_C(X, 64)

namespace efla {

// euler: alpha = beta (explicit Euler step) instead of the exact-flow alpha.
hipError_t dispatch_coef(bool bf16, int dk, const void *k, const float *beta, float *alpha,
                         float *lambda, long n, bool euler, hipStream_t st);

// slots != NULL: token n = nh / H updates pool entry slots[n] of P (see
// decode_kernel for the rejection of repeated or out-of-range slots).
hipError_t dispatch_decode(bool bf16, int dk, int dv, const void *q, const void *k, const void *v,
                           const float *beta, float *S, void *o, long NH, bool euler,
                           hipStream_t st, const int *slots = nullptr, int N = 0, int H = 1,
                           int P = 0, int *err = nullptr);

// Packed sequences (the chunked kernels' varlen form).  Head h's L-token
// axis holds N sequences back to back, sequence n at [cu[n], cu[n+1]) (cu:
// device int32 [N+1], offsets clamped into [0, L]); chunks restart at each
// sequence's first token.  dispatch_packed_chunks writes cu_chunks[n] (n = 0
// .. N), the chunks of the sequences before n (capped at ceil(L/C) + N, the
// most that sequences that do not overlap can have); the UT transform then
// runs on H heads with one workgroup per chunk (A stored by token, [H, L,
// C]), and the scans on BH = N * H sequences (bh = seq * H + h).
hipError_t dispatch_packed_chunks(const int *cu, int N, int L, int chunk, int *cu_chunks,
                                  hipStream_t st);

// cu_chunks != NULL: the packed form above, with BH = H.  alpha == NULL: the
// coefficients are formed inside from beta (euler: alpha = beta), lambda
// being the Gram diagonal the transform computes anyway; alpha_out and
// lambda_out (if given) then receive them, one float per token.
hipError_t dispatch_ut(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                       const void *v, const float *alpha, void *w, void *u, void *aqk, int BH,
                       int L, hipStream_t st, const int *cu = nullptr,
                       const int *cu_chunks = nullptr, int N = 0, int H = 1,
                       const float *beta = nullptr, bool euler = false,
                       float *alpha_out = nullptr, float *lambda_out = nullptr);

// cu != NULL: the packed form above.
hipError_t dispatch_scan(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                         const void *w, const void *u, const void *aqk, const float *S0, void *o,
                         float *SL, int BH, int L, int nw, hipStream_t st,
                         const int *cu = nullptr, int H = 1);

// The same scan split over L into G segments of seg_chunks chunks (the last
// may be shorter): segment maps (R [BH,G,dk,dv], P [BH,G,dk,dk]), their
// composition into entry states (Sin [BH,G,dk,dv]) and the segments replayed
// from them; o and S_L as from dispatch_scan.  Packed (cu != NULL): every
// sequence in G segments of ceil(its chunks / G) chunks (seg_chunks unused).
hipError_t dispatch_scan_segmented(bool bf16, int dk, int dv, int chunk, const void *q,
                                   const void *k, const void *w, const void *u, const void *aqk,
                                   const float *S0, void *o, float *SL, int BH, int L, int G,
                                   int seg_chunks, float *R, float *P, float *Sin, int nw,
                                   hipStream_t st, const int *cu = nullptr, int H = 1);

// Backward building blocks.  dispatch_scan_states runs the state scan for
// the entry state of every chunk only (states [BH, nchunks, dk, dv]; no o,
// no S_L).  dispatch_rscan walks the chunks backwards from dS_L (NULL = 0),
// writing every chunk's dS_out [BH, nchunks, dk, dv] and dE [BH, nchunks*chunk,
// dv] and, if dS0 is not NULL, dLoss/dS0 (fp32).  states, dS_out and dE are
// stored in the input dtype.  With G > 1 both scans run over G segments of
// seg_chunks chunks (maps R, P and composed boundary states Sin in fp32
// scratch, reused by the two).  dispatch_grad forms dq, dk, dv (dtype) and
// dbeta per chunk from them.
hipError_t dispatch_scan_states(bool bf16, int dk, int dv, int chunk, const void *q,
                                const void *k, const void *w, const void *u, const void *aqk,
                                const float *S0, void *states, int BH, int L, int nw, int G,
                                int seg_chunks, float *R, float *P, float *Sin, hipStream_t st);

hipError_t dispatch_rscan(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                          const void *w, const void *aqk, const void *dout, const float *dSL,
                          void *dSout, void *dE, float *dS0, int BH, int L, int nw, int G,
                          int seg_chunks, float *R, float *P, float *Sin, hipStream_t st);

hipError_t dispatch_grad(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                         const void *v, const void *dout, const float *beta, const float *alpha,
                         const float *lambda, const void *states, const void *dSout,
                         const void *dE, void *dq, void *dkp, void *dvp, float *dbeta, int BH,
                         int L, bool euler, hipStream_t st);

// dispatch_scan_states and dispatch_rscan (unsegmented) in one launch.
hipError_t dispatch_scan_pair(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                              const void *w, const void *u, const void *aqk, const float *S0,
                              void *states, const void *dout, const float *dSL, void *dSout,
                              void *dE, float *dS0, int BH, int L, int nw, hipStream_t st);

bool fused_supported(bool bf16, int dk, int dv, int chunk);

hipError_t dispatch_fused(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                          const void *v, const float *beta, const float *S0, void *o, float *SL,
                          int BH, int L, int nw, bool euler, hipStream_t st);

// Packed sequences: BH = N * H workgroup sequences, bh = seq * H + h; head h's
// tokens are an L-token axis holding the N sequences back to back, sequence
// seq at [cu[seq], cu[seq+1]) (cu: device int32 [N+1]).
hipError_t dispatch_fused_varlen(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                                 const void *v, const float *beta, const float *S0, void *o,
                                 float *SL, int BH, int L, const int *cu, int H, int nw, bool euler,
                                 hipStream_t st);

hipError_t launch_copy_state(const float *src, float *dst, long n, hipStream_t st);

}  // namespace efla
