// Per-chunk gradients of the chunkwise EFLA forward ("Exact Flow Linear
// Attention: Exact Solution from Continuous-Time Dynamics", Technical Summary,
// Methodology 3: the exact-flow update keeps the delta rule's chunkwise form;
// the pages train with it but print no backward).
//
// One chunk of C tokens, entry state S (d_k x d_v), D = diag(alpha):
//   Gamma = K K^T,  N = (I + D strictly_lower(Gamma))^{-1},  T = N D
//   X = V - K S         (the residuals v_t - S_{t-1}^T k_t, stacked)
//   E = T X,  O = Q S + (tril(Q K^T)) E,  S_out = S + K^T E.
// Given the chunk's dE = dLoss/dE and dS_out (both from the reverse scan;
// they and S are stored in the input dtype):
//   dX = T^T dE = D (N^T dE)                         dv = dX
//   dq = dO S^T + dA K,   dA = tril(dO E^T)
//   dk = -dX S^T + E dS_out^T + dA^T Q + dGam K + dGam^T K + 2 dlambda k
// and alpha enters through T = N D and through G = D strictly_lower(Gamma):
//   dalpha_j  = x_j . (N^T dE)_j                 (the D factor of T; x_j = row j of X)
//   dN  = dE (D X)^T,   dG = -strictly_lower(N^T dN N^T)
//   dalpha_i += sum_{j<i} dG_ij Gamma_ij,   dGam = D dG
//   dbeta = dalpha d alpha / d beta,   dlambda = dalpha d alpha / d lambda.
// fp32 throughout for fp32 inputs (fp32 MFMA 16x16x4).  For bf16 inputs
// every product with a d_k or d_v dimension rounds its operands to bf16 for
// bf16 MFMA, as the forward's bf16 path does; N and the C x C chain through
// it (N^T dN N^T) stay fp32.  One workgroup of 8 waves per
// chunk.  LDS holds K and two C x max(d_k, d_v) operand buffers in the input
// dtype and three fp32 C x C matrices (Gamma, N, dN); for bf16 inputs also a
// bf16 copy of N (later dGam) and dA in bf16, all of which only feed bf16
// MFMA.  The rows of dS_out go from the workspace straight into MFMA
// registers; the entry state does too for fp32 inputs and is staged through
// LDS for bf16 ones.  Wherever N's zeros make a block of a product exactly
// zero, the block is skipped.
#include <utility>

#include "efla_device.h"
#include "efla_launch.h"

namespace efla {

// d alpha / d beta and d alpha / d lambda.  With x = beta lambda:
// d alpha / d beta = e^{-x}; d alpha / d lambda = -beta^2 g(x) with
// g(x) = (1 - (1 + x) e^{-x}) / x^2 = sum_{n>=0} (-1)^n (n+1) x^n / (n+2)!,
// summed to n = 9 for |x| < 1/2 (the closed form cancels there), else the
// closed form.  Euler (alpha = beta): 1 and 0.
__device__ __forceinline__ void alpha_partials(int euler, float beta, float lambda, float &da_db,
                                               float &da_dl)
{
    if (euler) {
        da_db = 1.f;
        da_dl = 0.f;
        return;
    }
    const float x = beta * lambda;
    const float e = __builtin_amdgcn_exp2f(-x * 1.44269504088896341f);
    constexpr float c[10] = {1.f / 2,          -2.f / 6,         3.f / 24,         -4.f / 120,
                             5.f / 720,        -6.f / 5040,      7.f / 40320,      -8.f / 362880,
                             9.f / 3628800,    -10.f / 39916800};
    float p = c[9];
#pragma unroll
    for (int n = 8; n >= 0; --n) p = fmaf(p, x, c[n]);
    const float direct = (1.f - e - x * e) / (x * x);
    const float gx = fabsf(x) < 0.5f ? p : direct;
    da_db = e;
    da_dl = -beta * beta * gx;
}

// LDS of the gradient kernel.  K and the two C x max(d_k, d_v) operand
// buffers are held in the input dtype T: for bf16 inputs every reader of them
// feeds bf16 MFMA or rounds to the bf16 output, so storing them rounded
// changes no result and halves their LDS traffic.  Rows are padded by 16
// bytes.  The C x C matrices are fp32.
template <typename T, int DK, int DV, int C>
struct GradLayout {
    static constexpr int NW = 8;
    static constexpr int PAD = 16 / (int)sizeof(T);
    static constexpr int LDK = DK + PAD, LDV = DV + PAD, LDC = C + 4;
    static constexpr size_t kBytes = sizeof(T) * C * LDK, vBytes = sizeof(T) * C * LDV;
    static constexpr size_t ccBytes = sizeof(float) * C * LDC;
    static constexpr size_t dBytes = kBytes > vBytes ? kBytes : vBytes;
    // bf16 inputs: the entry state is staged through B1 (d_k x d_v) before V
    // is, and N has a bf16 copy (the operand of the products with d_v)
    static constexpr bool BF = is_bf16<T>;
    static constexpr int LDN = C + 8;
    static constexpr size_t sBytes = BF ? sizeof(T) * DK * LDV : 0;
    static constexpr size_t nbBytes = BF ? 2 * C * LDN : 0;
    // B1 also holds two fp32 C x C matrices (dA and N^T dN) once E is dead
    static constexpr size_t b1a = dBytes > 2 * ccBytes ? dBytes : 2 * ccBytes;
    static constexpr size_t b1Bytes = b1a > sBytes ? b1a : sBytes;
    static constexpr size_t offK = 0;
    static constexpr size_t offB1 = offK + kBytes;
    static constexpr size_t offB2 = offB1 + b1Bytes;
    static constexpr size_t offGam = offB2 + dBytes;
    static constexpr size_t offN = offGam + ccBytes;
    static constexpr size_t offD = offN + ccBytes;
    // alpha, lambda, beta, dlambda [C] and two [NW][C] tables of per-wave
    // partial sums of dalpha (summed in a fixed order: deterministic)
    static constexpr size_t offNb = offD + ccBytes;
    static constexpr size_t offVec = offNb + nbBytes;
    static constexpr size_t bytes = offVec + sizeof(float) * (4 + 2 * NW) * C;
    static_assert(kBytes % 16 == 0 && vBytes % 16 == 0 && ccBytes % 16 == 0 && nbBytes % 16 == 0,
                  "16-byte aligned buffers");
};

// bf16 MFMA on operands held in LDS or registers: an fp32 operand is rounded
// to bf16 as it is fed (fp32 accumulation), a bf16 one is read as it is; the
// fp32 inputs' path keeps fp32 MFMA.

// Four consecutive-k elements (idx, k .. k+3) of an LDS operand as bf16,
// idx = idx0 + l16: element (idx, k) at M[idx*ld + k] or, STRIDED, at
// M[k*ld + idx].  fp32: one 16-byte read or four 4-byte reads, rounded; bf16:
// one 8-byte read or one transposing read (every lane of the group must take
// part).
template <bool STRIDED>
__device__ __forceinline__ bf16x4 op4(const float *M, int ld, int idx0, int k)
{
    const int idx = idx0 + (threadIdx.x & 15);
    if constexpr (!STRIDED) {
        return to_bf16x4(*reinterpret_cast<const f32x4 *>(M + idx * ld + k));
    } else {
        return to_bf16x4(f32x4{M[k * ld + idx], M[(k + 1) * ld + idx], M[(k + 2) * ld + idx],
                               M[(k + 3) * ld + idx]});
    }
}
template <bool STRIDED>
__device__ __forceinline__ bf16x4 op4(const __bf16 *M, int ld, int idx0, int k)
{
    return run4_lds<STRIDED>(M, ld, idx0, k);
}

// Four elements of T in registers: bf16x4 for bf16, f32x4 for fp32.
template <typename T> struct QuadOf { using type = f32x4; };
template <> struct QuadOf<__bf16> { using type = bf16x4; };
template <typename T> using Quad = typename QuadOf<T>::type;

// out[mt] += A[16mt.., 0:16KT] * B, A in LDS, B as KT acc tiles (PERM map):
// the bf16 counterpart of mm_acc_b<float, ...>.  B is given in fp32 (rounded
// as it is fed) or already in bf16.
__device__ __forceinline__ bf16x4 as_bf16x4(f32x4 x) { return to_bf16x4(x); }
__device__ __forceinline__ bf16x4 as_bf16x4(bf16x4 x) { return x; }

template <int MT, int KT, bool LOWER, bool A_STRIDED, typename TA, typename TB>
__device__ __forceinline__ void mm_acc_b_bf16(f32x4 (&out)[MT], const TA *A, int lda,
                                              const TB (&Bacc)[KT])
{
    const int lane = threadIdx.x & 63, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < (KT + 1) / 2; ++s) {
        const bool two = 2 * s + 1 < KT;
        const bf16x8 b = cat(as_bf16x4(Bacc[2 * s]), two ? as_bf16x4(Bacc[2 * s + 1]) : to_bf16x4(zero4()));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (LOWER && 2 * s > mt) continue;
            const bf16x4 a1 = op4<A_STRIDED>(A, lda, 16 * mt, 32 * s + 4 * g);
            const bf16x4 a2 = two ? op4<A_STRIDED>(A, lda, 16 * mt, 32 * s + 16 + 4 * g) : to_bf16x4(zero4());
            out[mt] = mma(cat(a1, a2), b, out[mt]);
        }
    }
}

// acc += A[i0:i0+16, 0:K] * B[0:K, j0:j0+16], both in LDS (element (i,k) of
// A at A[i*lda+k], or A[k*lda+i] if A_STRIDED; (k,j) of B at B[j*ldb+k], or
// B[k*ldb+j] if B_STRIDED): the bf16 counterpart of mm_lds<float, ...>.
// k >= klim (rounded up to 32) is skipped.  K = 16: lane groups 2 and 3 of
// the 32-wide k-block lie past K; they read an in-range block (no lane may
// skip a transposing read) and zero it.
template <int K, bool A_STRIDED, bool B_STRIDED, typename TA, typename TB>
__device__ __forceinline__ f32x4 mm_lds_bf16(f32x4 acc, const TA *A, int lda, int i0,
                                             const TB *B, int ldb, int j0, int klim = K)
{
    const int lane = threadIdx.x & 63, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < (K + 31) / 32; ++s) {
        if (32 * s >= klim) break;
        const int k = 32 * s + 8 * g;
        const bool in = k < K;
        const int kr = in ? k : k - 16;
        bf16x8 a = cat(op4<A_STRIDED>(A, lda, i0, kr), op4<A_STRIDED>(A, lda, i0, kr + 4));
        bf16x8 b = cat(op4<B_STRIDED>(B, ldb, j0, kr), op4<B_STRIDED>(B, ldb, j0, kr + 4));
        const bf16x8 z = cat(to_bf16x4(zero4()), to_bf16x4(zero4()));
        a = in ? a : z;
        b = in ? b : z;
        acc = mma(a, b, acc);
    }
    return acc;
}

// The products with a d_k or d_v dimension, on bf16 MFMA for bf16 inputs and
// fp32 MFMA for fp32 inputs (whose operands are then all fp32).
template <typename T, int MT, int KT, bool LOWER = false, bool A_STRIDED = false, typename TA,
          typename TB>
__device__ __forceinline__ void mm_b(f32x4 (&out)[MT], const TA *A, int lda, const TB (&Bacc)[KT])
{
    if constexpr (is_bf16<T>) mm_acc_b_bf16<MT, KT, LOWER, A_STRIDED>(out, A, lda, Bacc);
    else mm_acc_b<float, MT, KT, LOWER, A_STRIDED>(out, A, lda, Bacc);
}

template <typename T, int K, bool A_STRIDED, bool B_STRIDED, typename TA, typename TB>
__device__ __forceinline__ f32x4 mm_t(f32x4 acc, const TA *A, int lda, int i0, const TB *B,
                                      int ldb, int j0, int klim = K)
{
    if constexpr (is_bf16<T>)
        return mm_lds_bf16<K, A_STRIDED, B_STRIDED>(acc, A, lda, i0, B, ldb, j0, klim);
    else return mm_lds<float, K, A_STRIDED, B_STRIDED>(acc, A, lda, i0, B, ldb, j0, klim);
}

// Rows [0, valid) of a ROWS x COLS tile of T in LDS (row stride s_ld, 16-byte
// aligned rows) to global memory with 16-byte non-temporal stores (final
// outputs, not read again by the writer).
template <typename T, int ROWS, int COLS, int NT>
__device__ __forceinline__ void store_rows_nt(T *g, long g_ld, const T *s, int s_ld, int valid)
{
    constexpr int V = 16 / sizeof(T), VPR = COLS / V, N = ROWS * VPR;
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int j = 0; j < (N + NT - 1) / NT; ++j) {
        const int idx = (int)threadIdx.x + j * NT;
        const int row = idx / VPR, cv = idx % VPR;
        if ((N % NT == 0 || idx < N) && row < valid)
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t *>(s + row * s_ld + cv * V),
                                        reinterpret_cast<u32x4_t *>(g + row * g_ld + cv * V));
    }
}

// Sum over the 16 lanes of a lane group (one acc-tile row), by DPP moves
// within the row: pairs, then quads, then lane 0 adds lane 4 (a rotation of
// the row by 12) and lane 8 (by 8).  Lane 0 holds the butterfly sum
// ((x0 + x1) + (x2 + x3)) + ((x4 + x5) + (x6 + x7)) + (lanes 8 .. 15 alike);
// the other lanes hold partial sums.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf,
                                                              0xf, false));
}
__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp_mov<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    x += dpp_mov<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    x += dpp_mov<0x12C>(x);   // row_ror:12
    x += dpp_mov<0x128>(x);   // row_ror:8
    return x;
}

// Row broadcast within each 16-lane row of the wave: every lane receives
// lane I's x (DPP row_newbcast).
template <int I>
__device__ __forceinline__ float row_bcast(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + I,
                                                              0xf, 0xf, false));
}

// Column j = l16 of the diagonal block N_bb (rows b0 .. b0+15), by the
// right-looking substitution: once N[i][j] is known it is added into every
// later row's sum, sum_m += Gamma[m][i] N[i][j], with Gamma[m][i] taken from
// lane i, which holds column i of the block.  Each row's sum gets its terms
// in the order i = 0, 1, .. and the same fused multiply-adds as the
// left-looking loop  N[i][j] = delta_ij - alpha_i sum_{m<i} Gamma_im N[m][j].
template <int I>
__device__ __forceinline__ void diag_step(float (&acc)[16], const float (&gc)[16], const float (&al)[16],
                                          int j, float (&n)[16])
{
    n[I] = (I == j ? 1.f : 0.f) - al[I] * acc[I];
#pragma unroll
    for (int m = I + 1; m < 16; ++m) acc[m] = fmaf(row_bcast<I>(gc[m]), n[I], acc[m]);
}
template <int... I>
__device__ __forceinline__ void diag_steps(float (&acc)[16], const float (&gc)[16], const float (&al)[16],
                                           int j, float (&n)[16], std::integer_sequence<int, I...>)
{
    (diag_step<I>(acc, gc, al, j, n), ...);
}
template <bool BF>
__device__ __forceinline__ void diag_block_solve(const float *sGam, const float *sAl, float *sN,
                                                 __bf16 *sNb, int ldc, int ldn, int b0, int j)
{
    float gc[16], al[16], acc[16], n[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        gc[m] = sGam[(b0 + m) * ldc + b0 + j];   // Gamma[m][j], below the diagonal for m > j
        al[m] = sAl[b0 + m];
        acc[m] = 0.f;
    }
    diag_steps(acc, gc, al, j, n, std::make_integer_sequence<int, 16>{});
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        sN[(b0 + i) * ldc + b0 + j] = n[i];
        if constexpr (BF) sNb[(b0 + i) * ldn + b0 + j] = static_cast<__bf16>(n[i]);
    }
}

template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(512) void grad_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ dout, const float *__restrict__ beta, const float *__restrict__ alpha,
    const float *__restrict__ lambda, const T *__restrict__ states,
    const T *__restrict__ dSout, const T *__restrict__ dE, T *__restrict__ dq,
    T *__restrict__ dk, T *__restrict__ dv, float *__restrict__ dbeta, int L, int nchunks,
    int euler)
{
    using Lay = GradLayout<T, DK, DV, C>;
    constexpr int NW = Lay::NW, NT = 64 * NW, MC = C / 16, MK = DK / 16, MV = DV / 16;
    constexpr int LDK = Lay::LDK, LDV = Lay::LDV, LDC = Lay::LDC;
    constexpr int TPW = (MC * MC + NW - 1) / NW;   // C x C tiles per wave
    static_assert(MC <= 4 && NW == 8, "a wave's C x C tiles t, t + NW lie in distinct block rows");
    extern __shared__ __align__(16) char smem[];
    T *sK = reinterpret_cast<T *>(smem + Lay::offK);
    T *sB1 = reinterpret_cast<T *>(smem + Lay::offB1);
    T *sB2 = reinterpret_cast<T *>(smem + Lay::offB2);
    float *sGam = reinterpret_cast<float *>(smem + Lay::offGam);
    float *sN = reinterpret_cast<float *>(smem + Lay::offN);
    float *sD = reinterpret_cast<float *>(smem + Lay::offD);
    __bf16 *sNb = reinterpret_cast<__bf16 *>(smem + Lay::offNb);   // bf16 inputs only
    T *sS = sB1;                                                      // bf16 inputs: S, phases 0-1
    constexpr bool BF = Lay::BF;
    constexpr int LDN = Lay::LDN;
    float *sAl = reinterpret_cast<float *>(smem + Lay::offVec);
    float *sLam = sAl + C, *sBeta = sAl + 2 * C, *sDl = sAl + 3 * C;
    float *sPT = sAl + 4 * C, *sPG = sPT + NW * C;   // [NW][C] partials of dalpha
    float *sdA = reinterpret_cast<float *>(smem + Lay::offB1), *sZ = sdA + C * LDC;   // B1 once E is dead
    // bf16 inputs: dA (in B1) and dGam (in N's bf16 copy, free after the
    // X / E / Y phase) are stored in bf16 -- they only feed bf16 MFMA
    __bf16 *sdAb = reinterpret_cast<__bf16 *>(smem + Lay::offB1), *sdGb = sNb;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, g = lane >> 4;
    const int bh = blockIdx.x / nchunks, c = blockIdx.x - bh * nchunks;
    const long tok0 = (long)bh * L + (long)c * C;
    const int valid = min(C, L - c * C);
    const T *Sst = states + ((long)bh * nchunks + c) * DK * DV;
    const T *dSo = dSout + ((long)bh * nchunks + c) * DK * DV;
    const T *dEg = dE + ((long)bh * nchunks * C + (long)c * C) * DV;

    // ---- every input in flight at once, in the order of first use: the
    // per-token scalars and K (Gamma, N), the entry state, V and dE, the rows
    // of dS_out (and for fp32 of S), then dO and Q.  Loads return in order and
    // the barriers below wait for LDS only, so each wait covers just the loads
    // a phase needs and the rest stay in flight under the earlier phases.
    float al0 = 0.f, la0 = 0.f, be0 = 0.f;
    if (tid < C && tid < valid) {
        al0 = alpha[tok0 + tid];
        la0 = lambda[tok0 + tid];
        be0 = beta[tok0 + tid];
    }
    TileRegs<T, C, DK, NT> rK, rQ;
    TileRegs<T, C, DV, NT> rV, rO;
    TileRegs<T, C, DV, NT> rE;
    TileRegs<T, DK, DV, NT> rS;
    rK.load(k + tok0 * DK, DK, valid);
    // The entry state S: the columns 16 wv .. of this wave (the B operand of
    // K S, tiles kt = rows 16 kt ..) and its rows 16 wv + l16 (of S^T).
    // bf16: staged through LDS with 16-byte loads (then one transposing or
    // 8-byte read per tile); fp32: straight from memory, kept in the input
    // dtype until the phase that reads them (widening them here would wait
    // for the loads at once).
    T Sr[MK][4];
    Quad<T> Sb[MK], SinT[MV], dSoT[MV];
    if constexpr (BF) {
        rS.load(Sst, DV, DK);
    } else if (MV >= NW || wv < MV) {
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int r = 0; r < 4; ++r) Sr[mk][r] = Sst[(16 * mk + 4 * g + r) * DV + 16 * wv + l16];
    }
    if constexpr (BF) __builtin_amdgcn_sched_barrier(0);   // keep the issue order of the load groups
    rV.load(v + tok0 * DV, DV, valid);
    rE.load(dEg, DV, valid);
    if constexpr (BF) __builtin_amdgcn_sched_barrier(0);
    // rows a = 16 wv + l16 of S and dS_out: B operands (k = d_v, j = a).
    // fp32: issued after the X / E / Y phase, whose registers they would crowd
    auto load_rows = [&]() {
        if (MK >= NW || wv < MK) {
            const int a = 16 * wv + l16;
#pragma unroll
            for (int kt = 0; kt < MV; ++kt) {
                if constexpr (!BF) SinT[kt] = *reinterpret_cast<const Quad<T> *>(Sst + a * DV + 16 * kt + 4 * g);
                dSoT[kt] = *reinterpret_cast<const Quad<T> *>(dSo + a * DV + 16 * kt + 4 * g);
            }
        }
    };
    if constexpr (BF) load_rows();
    if constexpr (BF) __builtin_amdgcn_sched_barrier(0);
    rO.load(dout + tok0 * DV, DV, valid);
    rQ.load(q + tok0 * DK, DK, valid);
    if constexpr (BF) __builtin_amdgcn_sched_barrier(0);
    rK.store(sK, LDK, valid);
    if constexpr (BF) rS.store(sS, LDV, DK);

    // ---- per-token scalars; Gamma and N -------------------------------------
    for (int e = tid; e < C * LDC; e += NT) sN[e] = 0.f;
    if constexpr (BF)
        for (int e = tid; e < C * LDN / 2; e += NT) reinterpret_cast<unsigned *>(sNb)[e] = 0u;
    if (tid < C) {
        sAl[tid] = al0;
        sLam[tid] = la0;
        sBeta[tid] = be0;
    }
    for (int e = tid; e < 2 * NW * C; e += NT) sPT[e] = 0.f;
    lds_barrier();
    if constexpr (BF) {   // S from its LDS staging (B1 takes V at the end of the N phases)
        if (MV >= NW || wv < MV) {
#pragma unroll
            for (int kt = 0; kt < MK; ++kt) Sb[kt] = run4_lds<true>(sS, LDV, 16 * wv, 16 * kt + 4 * g);
        }
        if (MK >= NW || wv < MK) {
#pragma unroll
            for (int kt = 0; kt < MV; ++kt) SinT[kt] = run4_lds<false>(sS, LDV, 16 * wv, 16 * kt + 4 * g);
        }
    }
    for (int t = wv; t < MC * MC; t += NW) {
        const int it = t / MC, jt = t - it * MC;
        if (jt > it) continue;
        const f32x4 acc = mm_t<T, DK, false, false>(zero4(), sK, LDK, 16 * it, sK, LDK, 16 * jt);   // exact products
#pragma unroll
        for (int r = 0; r < 4; ++r) sGam[(16 * it + 4 * g + r) * LDC + 16 * jt + l16] = acc[r];
    }
    lds_barrier();
    // diagonal 16x16 blocks: N_ij = delta_ij - alpha_i sum_{m<i} Gamma_im N_mj,
    // lane group g solving block g, lane j its column j
    if (wv == 0 && g < MC) diag_block_solve<BF>(sGam, sAl, sN, sNb, LDC, LDN, 16 * g, l16);
    lds_barrier();
    // blocks below: N_IJ = -N_II D_I sum_{M=J}^{I-1} Gamma_IM N_MJ.  Wave J
    // solves column block J right-looking: once N_MJ is known its term goes
    // into the sums of every later block row at once (independent MFMAs), and
    // it stays in registers in the accumulator layout (rows 4g + r of column
    // l16), the B operand of those products when a lane's four MFMAs take
    // k = 4g + r.  A column needs only its own and the diagonal blocks, so the
    // columns proceed side by side with one barrier at the end; every wave
    // then stages V and dE (S's staging in B1 was read before the last barrier).
    if (wv < MC - 1) {
        constexpr int NB = MC > 1 ? MC - 1 : 1;
        const int bj = wv, nb = MC - 1 - bj;   // blocks below the diagonal in column bj
        float gv[NB][NB][4];   // Gamma_{bj+1+d, bj+m}, m <= d: row l16, k = 4g + r
#pragma unroll
        for (int d = 0; d < MC - 1; ++d)
#pragma unroll
            for (int m = 0; m <= d; ++m) {
                const int bi = min(bj + 1 + d, MC - 1), bm = min(bj + m, MC - 1);
#pragma unroll
                for (int r = 0; r < 4; ++r) gv[d][m][r] = sGam[(16 * bi + l16) * LDC + 16 * bm + 4 * g + r];
            }
        f32x4 nb_reg, p[NB];
#pragma unroll
        for (int r = 0; r < 4; ++r) nb_reg[r] = sN[(16 * bj + 4 * g + r) * LDC + 16 * bj + l16];
#pragma unroll
        for (int d = 0; d < MC - 1; ++d) p[d] = zero4();
#pragma unroll
        for (int m = 0; m < MC - 1; ++m) {
            if (m >= nb) break;
#pragma unroll
            for (int d = m; d < MC - 1; ++d)
                if (d < nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) p[d] = mma(gv[d][m][r], nb_reg[r], p[d]);
            const int bn = bj + m + 1;   // block row bn's sum is complete
#pragma unroll
            for (int r = 0; r < 4; ++r) p[m][r] *= sAl[16 * bn + 4 * g + r];
            const f32x4 nnn = *reinterpret_cast<const f32x4 *>(sN + (16 * bn + l16) * LDC + 16 * bn + 4 * g);
            f32x4 x = zero4();
#pragma unroll
            for (int r = 0; r < 4; ++r) x = mma(nnn[r], p[m][r], x);
            nb_reg = -x;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sN[(16 * bn + 4 * g + r) * LDC + 16 * bj + l16] = nb_reg[r];
                if constexpr (BF) sNb[(16 * bn + 4 * g + r) * LDN + 16 * bj + l16] = static_cast<__bf16>(nb_reg[r]);
            }
        }
    }
    rV.store(sB1, LDV, valid);   // V and dE to LDS, for the first phase that reads them
    rE.store(sB2, LDV, valid);
    lds_barrier();

    // ---- per d_v column tile (wave wv owns columns 16wv .. 16wv+15) ----------
    f32x4 E[MC], dX[MC];
    if (wv < MV) {
        const int col = 16 * wv + l16;
        f32x4 X[MC], DXv[MC], dEc[MC], Y[MC];
#pragma unroll
        for (int mt = 0; mt < MC; ++mt) {
            X[mt] = zero4();
            if constexpr (BF) {   // rows 16 mt + 4 g + r of column col: one transposing read
                const bf16x4 e4 = run4_lds<true>(sB2, LDV, 16 * wv, 16 * mt + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) dEc[mt][r] = to_f32(e4[r]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) dEc[mt][r] = to_f32(sB2[(16 * mt + 4 * g + r) * LDV + col]);
            }
        }
        if constexpr (!BF) {
#pragma unroll
            for (int mk = 0; mk < MK; ++mk) Sb[mk] = Quad<T>{Sr[mk][0], Sr[mk][1], Sr[mk][2], Sr[mk][3]};
        }
        mm_b<T, MC, MK>(X, sK, LDK, Sb);   // K S
#pragma unroll
        for (int mt = 0; mt < MC; ++mt) {
            f32x4 vv;
            if constexpr (BF) {
                const bf16x4 v4 = run4_lds<true>(sB1, LDV, 16 * wv, 16 * mt + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) vv[r] = to_f32(v4[r]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) vv[r] = to_f32(sB1[(16 * mt + 4 * g + r) * LDV + col]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * mt + 4 * g + r;
                X[mt][r] = vv[r] - X[mt][r];   // V - K S
                DXv[mt][r] = sAl[row] * X[mt][r];
            }
            E[mt] = zero4();
            Y[mt] = zero4();
        }
        if constexpr (BF) {
            mm_b<T, MC, MC, true, false>(E, sNb, LDN, DXv);   // E = N (D X)
            mm_b<T, MC, MC, false, true>(Y, sNb, LDN, dEc);   // Y = N^T dE
        } else {
            mm_b<T, MC, MC, true, false>(E, sN, LDC, DXv);
            mm_b<T, MC, MC, false, true>(Y, sN, LDC, dEc);
        }
#pragma unroll
        for (int mt = 0; mt < MC; ++mt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * mt + 4 * g + r;
                dX[mt][r] = sAl[row] * Y[mt][r];
                const float part = row16_sum(X[mt][r] * Y[mt][r]);
                if (l16 == 0) sPT[wv * C + row] = part;
                sB1[row * LDV + col] = from_f32<T>(DXv[mt][r]);   // dE is already in B2
            }
        }
    }
    if constexpr (!BF) load_rows();
    lds_barrier();
    // dN = dE (D X)^T on and below the diagonal blocks (zero above)
    for (int t = wv; t < MC * MC; t += NW) {
        const int it = t / MC, jt = t - it * MC;
        f32x4 acc = zero4();
        if (jt <= it) acc = mm_t<T, DV, false, false>(zero4(), sB2, LDV, 16 * it, sB1, LDV, 16 * jt);
#pragma unroll
        for (int r = 0; r < 4; ++r) sD[(16 * it + 4 * g + r) * LDC + 16 * jt + l16] = acc[r];
    }
    lds_barrier();
    if (wv < MV) {
        const int col = 16 * wv + l16;
#pragma unroll
        for (int mt = 0; mt < MC; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * mt + 4 * g + r;
                sB1[row * LDV + col] = from_f32<T>(E[mt][r]);
                sB2[row * LDV + col] = from_f32<T>(dX[mt][r]);
            }
    }
    lds_barrier();
    store_rows_nt<T, C, DV, NT>(dv + tok0 * DV, DV, sB2, LDV, valid);   // dv = dX

    // ---- per d_k column tile (wave wv owns output columns 16wv .. 16wv+15) ---
    f32x4 dQw[MC], dKw[MC];
#pragma unroll
    for (int mt = 0; mt < MC; ++mt) {
        dQw[mt] = zero4();
        dKw[mt] = zero4();
    }
    if (wv < MK) {
        f32x4 t1[MC];
#pragma unroll
        for (int mt = 0; mt < MC; ++mt) t1[mt] = zero4();
        mm_b<T, MC, MV>(t1, sB2, LDV, SinT);    // dX S^T
        mm_b<T, MC, MV>(dKw, sB1, LDV, dSoT);   // E dS_out^T
#pragma unroll
        for (int mt = 0; mt < MC; ++mt) dKw[mt] -= t1[mt];
    }
    lds_barrier();
    rO.store(sB2, LDV, valid);
    lds_barrier();
    if (wv < MK) mm_b<T, MC, MV>(dQw, sB2, LDV, SinT);   // dO S^T
    // dA = tril(dO E^T), diagonal included
    f32x4 dAr[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = wv + u * NW;
        const int it = t / MC, jt = t - it * MC;
        dAr[u] = zero4();
        if (t < MC * MC && jt <= it) {
            dAr[u] = mm_t<T, DV, false, false>(zero4(), sB2, LDV, 16 * it, sB1, LDV, 16 * jt);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (16 * jt + l16 > 16 * it + 4 * g + r) dAr[u][r] = 0.f;
        }
    }
    lds_barrier();
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = wv + u * NW;
        if (t < MC * MC) {
            const int it = t / MC, jt = t - it * MC;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (BF) sdAb[(16 * it + 4 * g + r) * LDN + 16 * jt + l16] = static_cast<__bf16>(dAr[u][r]);
                else sdA[(16 * it + 4 * g + r) * LDC + 16 * jt + l16] = dAr[u][r];
            }
        }
    }
    rQ.store(sB2, LDK, valid);
    // Z = N^T dN, only its tiles on and below the diagonal (the ones dG
    // reads).  Row p of N is zero past p, so tile row it sums over p >= 16 it
    // only (the products skipped are exact zeros: the sums are unchanged).
    // Lower tile u (row-major) goes to wave u, then to wave 2 NW - 1 - u, so
    // the long rows pair with the short ones.
    constexpr int NZ = MC * (MC + 1) / 2;
    static_assert(NZ <= 2 * NW, "two lower tiles of Z per wave at most");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int u = h == 0 ? wv : 2 * NW - 1 - wv;
        if (u < NZ) {
            int it = 0;
            while ((it + 1) * (it + 2) / 2 <= u) ++it;
            const int jt = u - it * (it + 1) / 2;
            const f32x4 acc = mm_lds<float, C, true, true>(zero4(), sN + 16 * it * LDC, LDC, 16 * it,
                                                           sD + 16 * it * LDC, LDC, 16 * jt, C - 16 * it);
#pragma unroll
            for (int r = 0; r < 4; ++r) sZ[(16 * it + 4 * g + r) * LDC + 16 * jt + l16] = acc[r];
        }
    }
    lds_barrier();
    if (wv < MK) {
#pragma unroll
        for (int mt = 0; mt < MC; ++mt) {
            // dq += dA K;  dk += dA^T Q
            if constexpr (BF) {
                dQw[mt] = mm_t<T, C, false, true>(dQw[mt], sdAb, LDN, 16 * mt, sK, LDK, 16 * wv, 16 * mt + 16);
                dKw[mt] = mm_t<T, C, true, true>(dKw[mt], sdAb, LDN, 16 * mt, sB2, LDK, 16 * wv);
            } else {
                dQw[mt] = mm_t<T, C, false, true>(dQw[mt], sdA, LDC, 16 * mt, sK, LDK, 16 * wv, 16 * mt + 16);
                dKw[mt] = mm_t<T, C, true, true>(dKw[mt], sdA, LDC, 16 * mt, sB2, LDK, 16 * wv);
            }
        }
    }
    // dG = -strictly_lower(Z N^T); dalpha_i += sum_j dG_ij Gamma_ij; dGam = D dG
    f32x4 dGr[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = wv + u * NW;
        const int it = t / MC, jt = t - it * MC;
        dGr[u] = zero4();
        if (t < MC * MC && jt <= it) {
            // N^T is zero past column 16 jt + 15 of tile column jt: k < 16 (jt + 1)
            const f32x4 acc = mm_lds<float, C, false, false>(zero4(), sZ, LDC, 16 * it, sN, LDC, 16 * jt,
                                                             16 * jt + 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * it + 4 * g + r, cl = 16 * jt + l16;
                const float dg = cl < row ? -acc[r] : 0.f;
                // one tile per row block per wave (t and t + NW lie >= 2 block rows apart)
                const float part = row16_sum(dg * sGam[row * LDC + cl]);
                if (l16 == 0) sPG[wv * C + row] = part;
                dGr[u][r] = sAl[row] * dg;
            }
        }
    }
    lds_barrier();   // every read of dN (Z) and of dA, Q above is done
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = wv + u * NW;
        if (t < MC * MC) {
            const int it = t / MC, jt = t - it * MC;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (BF) sdGb[(16 * it + 4 * g + r) * LDN + 16 * jt + l16] = static_cast<__bf16>(dGr[u][r]);
                else sD[(16 * it + 4 * g + r) * LDC + 16 * jt + l16] = dGr[u][r];
            }
        }
    }
    lds_barrier();
    if (tid < C) {
        float da_db, da_dl;
        alpha_partials(euler, sBeta[tid], sLam[tid], da_db, da_dl);
        float da = 0.f;
        for (int w = 0; w < NW; ++w) da += sPT[w * C + tid];
        for (int w = 0; w < NW; ++w) da += sPG[w * C + tid];
        if (tid < valid) dbeta[tok0 + tid] = da * da_db;
        sDl[tid] = da * da_dl;
    }
    if (wv < MK) {
#pragma unroll
        for (int mt = 0; mt < MC; ++mt) {
            // dk += dGam K + dGam^T K
            if constexpr (BF) {
                dKw[mt] = mm_t<T, C, false, true>(dKw[mt], sdGb, LDN, 16 * mt, sK, LDK, 16 * wv, 16 * mt + 16);
                dKw[mt] = mm_t<T, C, true, true>(dKw[mt], sdGb, LDN, 16 * mt, sK, LDK, 16 * wv);
            } else {
                dKw[mt] = mm_t<T, C, false, true>(dKw[mt], sD, LDC, 16 * mt, sK, LDK, 16 * wv, 16 * mt + 16);
                dKw[mt] = mm_t<T, C, true, true>(dKw[mt], sD, LDC, 16 * mt, sK, LDK, 16 * wv);
            }
        }
    }
    lds_barrier();   // B1 and B2 are free: stage dq, dk for 16-byte stores
    if (wv < MK) {
        const int a = 16 * wv + l16;
#pragma unroll
        for (int mt = 0; mt < MC; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * mt + 4 * g + r;
                sB1[row * LDK + a] = from_f32<T>(dQw[mt][r]);
                sB2[row * LDK + a] = from_f32<T>(dKw[mt][r] + 2.f * sDl[row] * to_f32(sK[row * LDK + a]));
            }
    }
    lds_barrier();
    store_rows_nt<T, C, DK, NT>(dq + tok0 * DK, DK, sB1, LDK, valid);
    store_rows_nt<T, C, DK, NT>(dk + tok0 * DK, DK, sB2, LDK, valid);
}

template <typename T, int DK, int DV, int C>
hipError_t launch_grad(const void *q, const void *k, const void *v, const void *dout,
                       const float *beta, const float *alpha, const float *lambda,
                       const void *states, const void *dSout, const void *dE, void *dq,
                       void *dk, void *dv, float *dbeta, int BH, int L, bool euler, hipStream_t st)
{
    using Lay = GradLayout<T, DK, DV, C>;
    static_assert(Lay::bytes <= 160 * 1024, "gradient kernel LDS");
    const int nchunks = (L + C - 1) / C;
    if (BH == 0 || nchunks == 0) return hipSuccess;
    const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&grad_kernel<T, DK, DV, C>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((grad_kernel<T, DK, DV, C>), dim3((unsigned)(BH * nchunks)), dim3(64 * Lay::NW),
                       Lay::bytes, st, static_cast<const T *>(q), static_cast<const T *>(k),
                       static_cast<const T *>(v), static_cast<const T *>(dout), beta, alpha, lambda,
                       static_cast<const T *>(states), static_cast<const T *>(dSout),
                       static_cast<const T *>(dE), static_cast<T *>(dq), static_cast<T *>(dk),
                       static_cast<T *>(dv), dbeta, L, nchunks, (int)euler);
    return hipGetLastError();
}

hipError_t dispatch_grad(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                         const void *v, const void *dout, const float *beta, const float *alpha,
                         const float *lambda, const void *states, const void *dSout,
                         const void *dE, void *dq, void *dkp, void *dvp, float *dbeta, int BH,
                         int L, bool euler, hipStream_t st)
{
#define CASE(DKV, DVV, CC)                                                                      \
    if (dk == DKV && dv == DVV && chunk == CC)                                                  \
        return bf16 ? launch_grad<__bf16, DKV, DVV, CC>(q, k, v, dout, beta, alpha, lambda,     \
                                                        states, dSout, dE, dq, dkp, dvp, dbeta, \
                                                        BH, L, euler, st)                       \
                    : launch_grad<float, DKV, DVV, CC>(q, k, v, dout, beta, alpha, lambda,      \
                                                       states, dSout, dE, dq, dkp, dvp, dbeta,  \
                                                       BH, L, euler, st);
    EFLA_SHAPE_CASES(CASE)
#undef CASE
    return hipErrorInvalidValue;
}

}  // namespace efla
