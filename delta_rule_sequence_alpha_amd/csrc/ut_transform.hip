// Per-chunk UT transform (the chunkwise WY/UT scheme that "Exact Flow Linear
// Attention: Exact Solution from Continuous-Time Dynamics", Technical Summary,
// Methodology 3, says the exact-flow update keeps).
//
// For one chunk of C tokens with keys K, values V, queries Q and coefficients
// a = alpha, writing the update as S_r = S_{r-1} + k_r e_r^T with
// e_r = a_r (v_r - S_{r-1}^T k_r) and stacking e_r^T into E gives
//   (D^{-1} + strictly_lower(K K^T)) E = V - K S,   D = diag(a),
// so with T = (I + strictly_lower(D K K^T))^{-1} D, W = T K, U = T V:
//   E = U - W S.
// T is formed here without dividing by alpha:
//   T[i][j] = a_i (delta_ij - sum_{j<=m<i} (k_i.k_m) T[m][j]),
// by substitution inside each 16x16 diagonal block and by block substitution
//   T_ij = -T_ii sum_{m=j}^{i-1} G_im T_mj   (G = K K^T)
// below it, all in fp32.  ||T||_2 <= max beta in the chunk for beta >= 0, so the
// substitution works on bounded quantities.
#include "efla_device.h"
#include "efla_launch.h"

namespace efla {

template <typename T, int DK, int DV, int C>
struct UtLayout {
    static constexpr int PADE = is_bf16<T> ? 8 : 4;   // 16 bytes of row padding
    static constexpr int LDK = DK + PADE, LDV = DV + PADE;
    static constexpr int LDG = C + 1;                  // fp32, scalar access only
    static constexpr int LDTB = C + PADE;              // T converted to T-type
    // Q is only needed for A = tril(Q K^T), V only for U = T V: they share a
    // buffer (V waits in registers), which keeps bf16 chunks of 64 tokens at
    // d = 128 within two workgroups per CU.  K's buffer later stages W, the
    // Q/V buffer U, for 16-byte stores.
    static constexpr int LDQV = LDK > LDV ? LDK : LDV;
    static constexpr size_t offK = 0;
    static constexpr size_t offQ = offK + sizeof(T) * C * LDK;
    static constexpr size_t offV = offQ;
    static constexpr size_t offG = offQ + sizeof(T) * C * LDQV;
    static constexpr size_t offT = offG + sizeof(float) * C * LDG;
    static constexpr size_t offTb = offT + sizeof(float) * C * LDG;
    static constexpr size_t offA = offTb + (is_bf16<T> ? sizeof(T) * C * LDTB : 0);
    static constexpr size_t bytes = offA + sizeof(float) * C;
};

template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(256) void ut_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                 const T *__restrict__ v,
                                                 const float *__restrict__ alpha,
                                                 T *__restrict__ w, T *__restrict__ u,
                                                 T *__restrict__ aqk, int L, int nchunks)
{
    using Lay = UtLayout<T, DK, DV, C>;
    constexpr int MC = C / 16;
    constexpr bool BF = is_bf16<T>;
    extern __shared__ __align__(16) char smem[];
    T *sK = reinterpret_cast<T *>(smem + Lay::offK);
    T *sQ = reinterpret_cast<T *>(smem + Lay::offQ);
    T *sV = reinterpret_cast<T *>(smem + Lay::offV);
    float *sG = reinterpret_cast<float *>(smem + Lay::offG);
    float *sT = reinterpret_cast<float *>(smem + Lay::offT);
    T *sTb = reinterpret_cast<T *>(smem + Lay::offTb);
    float *sAl = reinterpret_cast<float *>(smem + Lay::offA);

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
    const int bh = blockIdx.x / nchunks, c = blockIdx.x - bh * nchunks;
    const long tok0 = (long)bh * L + (long)c * C;
    const int valid = min(C, L - c * C);

    // every load of the chunk in flight before the first LDS store
    TileRegs<T, C, DK, 256> tk, tq;
    TileRegs<T, C, DV, 256> tv;
    tk.load(k + tok0 * DK, DK, valid);
    tq.load(q + tok0 * DK, DK, valid);
    tv.load(v + tok0 * DV, DV, valid);
    tk.store(sK, Lay::LDK, valid);
    tq.store(sQ, Lay::LDK, valid);
    for (int i = threadIdx.x; i < C * Lay::LDG; i += 256) sT[i] = 0.f;
    for (int i = threadIdx.x; i < C; i += 256) sAl[i] = (i < valid) ? alpha[tok0 + i] : 0.f;
    __syncthreads();

    // Gram tiles G = K K^T (lower incl. diagonal, fp32 into LDS) and A = tril(Q K^T)
    // (written to global; tiles above the diagonal are written as zeros).
    T *aq = aqk + ((long)bh * nchunks + c) * C * C;
    for (int t = wv; t < 2 * MC * MC; t += 4) {
        const bool gram = t < MC * MC;
        const int tt = gram ? t : t - MC * MC;
        const int it = tt / MC, jt = tt - it * MC;
        if (gram) {
            if (jt > it) continue;
            const f32x4 acc = mm_lds<T, DK, false, false>(zero4(), sK, Lay::LDK, 16 * it, sK,
                                                          Lay::LDK, 16 * jt);
#pragma unroll
            for (int r = 0; r < 4; ++r) sG[(16 * it + 4 * g + r) * Lay::LDG + 16 * jt + l16] = acc[r];
        } else {
            f32x4 acc = zero4();
            if (jt <= it)
                acc = mm_lds<T, DK, false, false>(zero4(), sQ, Lay::LDK, 16 * it, sK, Lay::LDK,
                                                  16 * jt);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * it + 4 * g + r, col = 16 * jt + l16;
                aq[row * C + col] = from_f32<T>(col <= row ? acc[r] : 0.f);
            }
        }
    }
    __syncthreads();

    // Diagonal 16x16 blocks of T by forward substitution: wave 0, lane group b
    // handles block b, lane l16 owns column l16 of it.
    if (wv == 0 && g < MC) {
        const int b0 = 16 * g, j = l16;
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = (i == j) ? 1.f : 0.f;
            const float *grow = sG + (b0 + i) * Lay::LDG + b0;
#pragma unroll
            for (int m = 0; m < i; ++m) acc = fmaf(-grow[m], t[m], acc);
            t[i] = sAl[b0 + i] * acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[(b0 + i) * Lay::LDG + b0 + j] = t[i];
    }
    __syncthreads();

    // Blocks below the diagonal, one block distance at a time (fp32 MFMA).
    for (int dist = 1; dist < MC; ++dist) {
        if (wv < MC - dist) {
            const int bi = dist + wv, bj = wv;
            f32x4 p = zero4();
            for (int m = bj; m < bi; ++m) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float a = sG[(16 * bi + l16) * Lay::LDG + 16 * m + 4 * s + g];
                    const float b = sT[(16 * m + 4 * s + g) * Lay::LDG + 16 * bj + l16];
                    p = mma(a, b, p);
                }
            }
            f32x4 x = zero4();
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float a = sT[(16 * bi + l16) * Lay::LDG + 16 * bi + 4 * g + r];
                x = mma(a, p[r], x);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sT[(16 * bi + 4 * g + r) * Lay::LDG + 16 * bj + l16] = -x[r];
        }
        __syncthreads();
    }

    const T *sTop = nullptr;   // T as the MFMA A operand
    int ldTop = 0;
    if constexpr (BF) {
        for (int i = threadIdx.x; i < C * C; i += 256) {
            const int r = i / C, cc = i - r * C;
            sTb[r * Lay::LDTB + cc] = from_f32<T>(sT[r * Lay::LDG + cc]);
        }
        sTop = sTb;
        ldTop = Lay::LDTB;
    } else {
        sTop = reinterpret_cast<const T *>(sT);
        ldTop = Lay::LDG;
    }
    tv.store(sV, Lay::LDV, valid);   // A = tril(Q K^T) is done with Q
    __syncthreads();

    // W = T K and U = T V (T lower triangular: k range of row tile mt is
    // [0, 16mt+16)).  Each product is staged in LDS over the operand it no
    // longer needs (W over K, U over V) and written with 16-byte stores.
    constexpr int NTK = DK / 16, NTV = DV / 16;
    constexpr int WPW = (MC * NTK + 3) / 4, UPW = (MC * NTV + 3) / 4;   // tiles per wave
    f32x4 acc[WPW > UPW ? WPW : UPW];
#pragma unroll
    for (int j = 0; j < WPW; ++j) {
        const int t = wv + 4 * j, mt = t / NTK, nt = t - mt * NTK;
        if (t < MC * NTK)
            acc[j] = mm_lds<T, C, false, true>(zero4(), sTop, ldTop, 16 * mt, sK, Lay::LDK, 16 * nt,
                                               16 * mt + 16);
    }
    __syncthreads();   // every read of K is done
#pragma unroll
    for (int j = 0; j < WPW; ++j) {
        const int t = wv + 4 * j, mt = t / NTK, nt = t - mt * NTK;
        if (t < MC * NTK)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sK[(16 * mt + 4 * g + r) * Lay::LDK + 16 * nt + l16] = from_f32<T>(acc[j][r]);
    }
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
        const int t = wv + 4 * j, mt = t / NTV, nt = t - mt * NTV;
        if (t < MC * NTV)
            acc[j] = mm_lds<T, C, false, true>(zero4(), sTop, ldTop, 16 * mt, sV, Lay::LDV, 16 * nt,
                                               16 * mt + 16);
    }
    __syncthreads();   // every read of V is done; W is staged
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
        const int t = wv + 4 * j, mt = t / NTV, nt = t - mt * NTV;
        if (t < MC * NTV)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sV[(16 * mt + 4 * g + r) * Lay::LDV + 16 * nt + l16] = from_f32<T>(acc[j][r]);
    }
    __syncthreads();
    store_rows_t<T, C, DK, 256>(w + tok0 * DK, DK, sK, Lay::LDK, valid);
    store_rows_t<T, C, DV, 256>(u + tok0 * DV, DV, sV, Lay::LDV, valid);
}

template <typename T, int DK, int DV, int C>
hipError_t launch_ut(const void *q, const void *k, const void *v, const float *alpha, void *w,
                     void *u, void *aqk, int BH, int L, hipStream_t st)
{
    using Lay = UtLayout<T, DK, DV, C>;
    const int nchunks = (L + C - 1) / C;
    if (BH == 0 || nchunks == 0) return hipSuccess;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&ut_kernel<T, DK, DV, C>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((ut_kernel<T, DK, DV, C>), dim3((unsigned)(BH * nchunks)), dim3(256),
                       Lay::bytes, st, static_cast<const T *>(q), static_cast<const T *>(k),
                       static_cast<const T *>(v), alpha, static_cast<T *>(w),
                       static_cast<T *>(u), static_cast<T *>(aqk), L, nchunks);
    return hipGetLastError();
}

hipError_t dispatch_ut(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                       const void *v, const float *alpha, void *w, void *u, void *aqk, int BH,
                       int L, hipStream_t st)
{
#define CASE(DKV, DVV, CC)                                                                      \
    if (dk == DKV && dv == DVV && chunk == CC)                                                  \
        return bf16 ? launch_ut<__bf16, DKV, DVV, CC>(q, k, v, alpha, w, u, aqk, BH, L, st)     \
                    : launch_ut<float, DKV, DVV, CC>(q, k, v, alpha, w, u, aqk, BH, L, st);
    EFLA_SHAPE_CASES(CASE)
#undef CASE
    return hipErrorInvalidValue;
}

}  // namespace efla
