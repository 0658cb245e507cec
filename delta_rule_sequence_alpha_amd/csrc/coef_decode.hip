// Per-token coefficient kernel and the single-token decode kernel.
//
// Coefficients ("Exact Flow Linear Attention: Exact Solution from
// Continuous-Time Dynamics", Technical Summary, Methodology 2-3):
//   lambda_t = |k_t|^2,  alpha_t = (1 - e^{-beta_t lambda_t}) / lambda_t.
// Decode step: the same update applied to one token,
//   S <- S + alpha k r^T with r = v - S^T k,  o = S_new^T q = S^T q + alpha (k.q) r.
// Both kernels take `euler`: alpha = beta, the explicit Euler step of the
// same ODE (the delta rule), for comparison with the exact flow.
#include "efla_device.h"
#include "efla_launch.h"

namespace efla {

// ---------------------------------------------------------------------------
// Coefficients: a group of LPT lanes per token, each lane reading 16 bytes of
// k; lambda is reduced across the group with butterfly shuffles.
template <typename T, int DK>
__global__ __launch_bounds__(256) void coef_kernel(const T *__restrict__ k,
                                                   const float *__restrict__ beta,
                                                   float *__restrict__ alpha,
                                                   float *__restrict__ lambda, long n_tokens,
                                                   int euler)
{
    constexpr int V = 16 / sizeof(T);
    constexpr int LPT = DK / V;                 // lanes per token (<= 64)
    constexpr int TPB = 256 / LPT;              // tokens per block
    const int sub = threadIdx.x % LPT;
    const long tok = (long)blockIdx.x * TPB + threadIdx.x / LPT;
    float acc = 0.f;
    if (tok < n_tokens) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(k + tok * DK + sub * V);
        const T *e = reinterpret_cast<const T *>(&raw);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const float x = to_f32(e[i]);
            acc = fmaf(x, x, acc);
        }
    }
#pragma unroll
    for (int off = LPT / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (tok < n_tokens && sub == 0) {
        alpha[tok] = update_alpha(euler, beta[tok], acc);
        if (lambda) lambda[tok] = acc;
    }
}

template <typename T, int DK>
hipError_t launch_coef(const void *k, const float *beta, float *alpha, float *lambda,
                       long n_tokens, bool euler, hipStream_t st)
{
    constexpr int LPT = DK / (16 / sizeof(T));
    constexpr int TPB = 256 / LPT;
    if (n_tokens == 0) return hipSuccess;
    const long blocks = (n_tokens + TPB - 1) / TPB;
    hipLaunchKernelGGL((coef_kernel<T, DK>), dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const T *>(k), beta, alpha, lambda, n_tokens, (int)euler);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode: one workgroup per (n,h).  Thread t owns a 4-column group c of S and
// the rows rg, rg+RG, ... ; S is loaded once with 128-bit reads into
// registers, reduced, updated and written back with 128-bit stores.
template <int DK, int DV>
struct DecodeShape {
    static constexpr int CG = DV / 4;                                    // column groups
    static constexpr int NT = (DK * DV / 4) >= 256 ? 256 : (DK * DV / 4);  // threads
    static constexpr int RG = NT / CG;                                   // row groups
    static constexpr int RPT = DK / RG;                                  // rows per thread
};

// Slot-indexed form (slots != NULL): token n's state is entry slots[n] of a
// pool of P sequences, nh = n * H + h.  A slot outside [0, P), or one that
// more than one token of the batch names, is rejected: its tokens leave the
// pool untouched, their outputs are NaN, and err (if given) is OR-ed with 2
// or 1.  Every thread of the workgroup takes the same decision (the slot is
// per token, the repeat test is reduced over the workgroup).
template <typename T, int DK, int DV>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT)) void decode_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ beta, float *__restrict__ S, T *__restrict__ o, int euler,
    const int *__restrict__ slots, int N, int H, int P, int *__restrict__ err)
{
    using Sh = DecodeShape<DK, DV>;
    constexpr int NT = Sh::NT, CG = Sh::CG, RG = Sh::RG, RPT = Sh::RPT;
    static_assert(RG * CG == NT && RPT * RG == DK, "decode shape");
    static_assert(NT >= DV, "one thread per output column of a rejected token");
    __shared__ float sk[DK], sq[DK], sv[DV];
    __shared__ float4 red_k[RG][CG], red_q[RG][CG];
    __shared__ float s_alpha, s_kq;

    const long nh = blockIdx.x;
    const int tid = threadIdx.x;
    long sidx = nh;   // the state this token updates
    if (slots) {
        const int n = (int)(nh / H), h = (int)(nh - (long)n * H);
        const int slot = slots[n];
        const int bad = slot < 0 || slot >= P;
        int rep = 0;
        for (int j = tid; j < N; j += NT) rep |= (j != n && slots[j] == slot);
        rep = __syncthreads_or(rep);
        if (bad || rep) {
            if (tid < DV) o[nh * DV + tid] = from_f32<T>(__builtin_nanf(""));
            if (tid == 0 && err) atomicOr(err, (bad ? 2 : 0) | (rep ? 1 : 0));
            return;
        }
        sidx = (long)slot * H + h;
    }
    for (int i = tid; i < DK; i += NT) {
        sk[i] = to_f32(k[nh * DK + i]);
        sq[i] = to_f32(q[nh * DK + i]);
    }
    for (int i = tid; i < DV; i += NT) sv[i] = to_f32(v[nh * DV + i]);

    const int c = tid % CG, rg = tid / CG;
    float4 *Sp = reinterpret_cast<float4 *>(S + sidx * DK * DV);
    float4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = Sp[(rg + i * RG) * CG + c];
    __syncthreads();

    if (tid < 64) {   // wave 0: lambda = |k|^2 and k.q
        float lam = 0.f, kq = 0.f;
        for (int i = tid; i < DK; i += 64) {
            lam = fmaf(sk[i], sk[i], lam);
            kq = fmaf(sk[i], sq[i], kq);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            lam += __shfl_xor(lam, off, 64);
            kq += __shfl_xor(kq, off, 64);
        }
        if (tid == 0) {
            s_alpha = update_alpha(euler, beta[nh], lam);
            s_kq = kq;
        }
    }

    float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float kr = sk[rg + i * RG], qr = sq[rg + i * RG];
        pk.x = fmaf(kr, s[i].x, pk.x); pk.y = fmaf(kr, s[i].y, pk.y);
        pk.z = fmaf(kr, s[i].z, pk.z); pk.w = fmaf(kr, s[i].w, pk.w);
        pq.x = fmaf(qr, s[i].x, pq.x); pq.y = fmaf(qr, s[i].y, pq.y);
        pq.z = fmaf(qr, s[i].z, pq.z); pq.w = fmaf(qr, s[i].w, pq.w);
    }
    red_k[rg][c] = pk;
    red_q[rg][c] = pq;
    __syncthreads();

    float4 tk = make_float4(0.f, 0.f, 0.f, 0.f), tq = tk;
#pragma unroll 8
    for (int j = 0; j < RG; ++j) {
        const float4 a = red_k[j][c], b = red_q[j][c];
        tk.x += a.x; tk.y += a.y; tk.z += a.z; tk.w += a.w;
        tq.x += b.x; tq.y += b.y; tq.z += b.z; tq.w += b.w;
    }
    const float al = s_alpha;
    // r = v - S^T k (columns 4c..4c+3); the update adds alpha k_i r_j
    const float4 r = make_float4(sv[4 * c + 0] - tk.x, sv[4 * c + 1] - tk.y,
                                 sv[4 * c + 2] - tk.z, sv[4 * c + 3] - tk.w);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float ak = al * sk[rg + i * RG];
        float4 x = s[i];
        x.x = fmaf(ak, r.x, x.x); x.y = fmaf(ak, r.y, x.y);
        x.z = fmaf(ak, r.z, x.z); x.w = fmaf(ak, r.w, x.w);
        // non-temporal: the new state is not read again by this launch, and
        // write-allocating it would evict the state still to be read (at
        // N = 512, 16 heads, d = 128: 6.74 vs 5.15 TB/s; at N = 256, where
        // the state fits the Infinity Cache, 6.68 vs 6.44 TB/s)
        __builtin_nontemporal_store(f32x4{x.x, x.y, x.z, x.w},
                                    reinterpret_cast<f32x4 *>(Sp) + (rg + i * RG) * CG + c);
    }
    if (rg == 0) {
        const float akq = al * s_kq;
        T *op = o + nh * DV + 4 * c;
        op[0] = from_f32<T>(fmaf(akq, r.x, tq.x));
        op[1] = from_f32<T>(fmaf(akq, r.y, tq.y));
        op[2] = from_f32<T>(fmaf(akq, r.z, tq.z));
        op[3] = from_f32<T>(fmaf(akq, r.w, tq.w));
    }
}

template <typename T, int DK, int DV>
hipError_t launch_decode(const void *q, const void *k, const void *v, const float *beta, float *S,
                         void *o, long NH, bool euler, const int *slots, int N, int H, int P,
                         int *err, hipStream_t st)
{
    if (NH == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_kernel<T, DK, DV>), dim3((unsigned)NH),
                       dim3(DecodeShape<DK, DV>::NT), 0, st, static_cast<const T *>(q),
                       static_cast<const T *>(k), static_cast<const T *>(v), beta, S,
                       static_cast<T *>(o), (int)euler, slots, N, H, P, err);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// S_L <- S0 (or zero) for sequences with no tokens.
__global__ void copy_state_kernel(const float *__restrict__ src, float *__restrict__ dst, long n)
{
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_copy_state(const float *src, float *dst, long n, hipStream_t st)
{
    if (n == 0 || src == dst) return hipSuccess;
    hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       src, dst, n);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dispatch over the supported (dtype, d) set.
#define EFLA_D_CASES(X) X(16) X(32) X(64) X(128)

hipError_t dispatch_coef(bool bf16, int dk, const void *k, const float *beta, float *alpha,
                         float *lambda, long n, bool euler, hipStream_t st)
{
#define CASE(D)                                                                              \
    if (dk == D)                                                                             \
        return bf16 ? launch_coef<__bf16, D>(k, beta, alpha, lambda, n, euler, st)           \
                    : launch_coef<float, D>(k, beta, alpha, lambda, n, euler, st);
    EFLA_D_CASES(CASE)
#undef CASE
    return hipErrorInvalidValue;
}

hipError_t dispatch_decode(bool bf16, int dk, int dv, const void *q, const void *k, const void *v,
                           const float *beta, float *S, void *o, long NH, bool euler,
                           hipStream_t st, const int *slots, int N, int H, int P, int *err)
{
#define CASE2(DKV, DVV)                                                                      \
    if (dk == DKV && dv == DVV)                                                              \
        return bf16 ? launch_decode<__bf16, DKV, DVV>(q, k, v, beta, S, o, NH, euler, slots,  \
                                                      N, H, P, err, st)                      \
                    : launch_decode<float, DKV, DVV>(q, k, v, beta, S, o, NH, euler, slots,   \
                                                     N, H, P, err, st);
#define CASE(D) CASE2(D, 16) CASE2(D, 32) CASE2(D, 64) CASE2(D, 128)
    EFLA_D_CASES(CASE)
#undef CASE
#undef CASE2
    return hipErrorInvalidValue;
}

}  // namespace efla
