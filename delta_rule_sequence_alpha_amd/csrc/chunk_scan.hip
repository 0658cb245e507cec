// Inter-chunk state scan of the chunkwise EFLA forward ("Exact Flow Linear
// Attention: Exact Solution from Continuous-Time Dynamics", Technical Summary,
// Methodology 3: the rank-1 update keeps the delta rule's chunkwise form).
//
// Per chunk with entry state S (d_k x d_v) and W, U, A = tril(Q K^T) from the
// UT transform:
//   E = U - W S            (the chunk's rank-1 corrections e_r stacked)
//   O = Q S + A E          (o_r = S_r^T q_r for every token of the chunk)
//   S <- S + K^T E         (state after the chunk)
//
// Columns of S evolve independently (the update multiplies S from the left
// only), so a workgroup owns a (sequence, 16*NW-column tile) and each wave
// owns 16 columns: all d_k rows of them stay in MFMA accumulators for the
// whole sequence, and every product above is wave-local.  The state feeds the
// next MFMA as its B operand straight from the accumulators (PERM map).
#include "efla_device.h"
#include "efla_launch.h"

namespace efla {

template <typename T, int DK, int DV, int C, int NW>
struct ScanLayout {
    static constexpr int PADE = is_bf16<T> ? 8 : 4;
    static constexpr int TV = 16 * NW;
    static constexpr int LDK = DK + PADE, LDC = C + PADE, LDU = TV + PADE;
    static constexpr size_t offW = 0;
    static constexpr size_t offQ = offW + sizeof(T) * C * LDK;
    static constexpr size_t offK = offQ + sizeof(T) * C * LDK;
    static constexpr size_t offA = offK + sizeof(T) * C * LDK;
    static constexpr size_t offU = offA + sizeof(T) * C * LDC;
    static constexpr size_t bytes = offU + sizeof(T) * C * LDU;
};

template <typename T, int DK, int DV, int C, int NW>
__global__ __launch_bounds__(64 * NW) void scan_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ w,
    const T *__restrict__ u, const T *__restrict__ aqk, const float *__restrict__ S0,
    T *__restrict__ o, float *__restrict__ SL, int L, int nchunks)
{
    using Lay = ScanLayout<T, DK, DV, C, NW>;
    constexpr int TV = Lay::TV, NTILE = DV / TV, MC = C / 16, MK = DK / 16;
    constexpr int NT = 64 * NW;
    extern __shared__ __align__(16) char smem[];
    T *sW = reinterpret_cast<T *>(smem + Lay::offW);
    T *sQ = reinterpret_cast<T *>(smem + Lay::offQ);
    T *sK = reinterpret_cast<T *>(smem + Lay::offK);
    T *sA = reinterpret_cast<T *>(smem + Lay::offA);
    T *sU = reinterpret_cast<T *>(smem + Lay::offU);

    int bh, tile;
    xcd_map(blockIdx.x, gridDim.x, NTILE, bh, tile);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
    const int col = tile * TV + 16 * wv + l16;   // this lane's state column

    f32x4 S[MK];
    const long sbase = (long)bh * DK * DV;
    if (S0) {   // one branch around all the loads, so they are in flight together
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int r = 0; r < 4; ++r) S[mk][r] = S0[sbase + (16 * mk + 4 * g + r) * DV + col];
    } else {
#pragma unroll
        for (int mk = 0; mk < MK; ++mk) S[mk] = zero4();
    }

    // The next chunk's tiles are loaded into registers while this chunk is
    // computed (chunks past the end re-load the last chunk, never stored).
    // Shapes whose tiles would not fit in registers load each tile at the top
    // of its chunk instead, one tile at a time.
    using RW = TileRegs<T, C, DK, NT>;
    using RU = TileRegs<T, C, TV, NT>;
    using RA = TileRegs<T, C, C, NT>;
    constexpr bool PREFETCH = 3 * RW::PER + RU::PER + RA::PER <= 40;
    RW rW, rQ, rK;
    RU rU;
    RA rA;
    auto load_all = [&](int cn) {
        cn = min(cn, nchunks - 1);
        const long t0 = (long)bh * L + (long)cn * C;
        const int vn = min(C, L - cn * C);
        rW.load(w + t0 * DK, DK, vn);
        rQ.load(q + t0 * DK, DK, vn);
        rK.load(k + t0 * DK, DK, vn);
        rU.load(u + t0 * DV + tile * TV, DV, vn);
        rA.load(aqk + ((long)bh * nchunks + cn) * C * C, C, C);
    };
    if constexpr (PREFETCH) load_all(0);

    for (int c = 0; c < nchunks; ++c) {
        const long tok0 = (long)bh * L + (long)c * C;
        const int valid = min(C, L - c * C);
        __syncthreads();   // the previous chunk is done with LDS
        if constexpr (PREFETCH) {
            rW.store(sW, Lay::LDK, valid);
            rQ.store(sQ, Lay::LDK, valid);
            rK.store(sK, Lay::LDK, valid);
            rU.store(sU, Lay::LDU, valid);
            rA.store(sA, Lay::LDC, C);
            load_all(c + 1);
        } else {
            RW t;
            t.load(w + tok0 * DK, DK, valid);
            t.store(sW, Lay::LDK, valid);
            t.load(q + tok0 * DK, DK, valid);
            t.store(sQ, Lay::LDK, valid);
            t.load(k + tok0 * DK, DK, valid);
            t.store(sK, Lay::LDK, valid);
            rU.load(u + tok0 * DV + tile * TV, DV, valid);
            rU.store(sU, Lay::LDU, valid);
            rA.load(aqk + ((long)bh * nchunks + c) * C * C, C, C);
            rA.store(sA, Lay::LDC, C);
        }
        __syncthreads();

        // E = U - W S
        f32x4 E[MC];
#pragma unroll
        for (int mt = 0; mt < MC; ++mt) E[mt] = zero4();
        mm_acc_b<T, MC, MK, false, false>(E, sW, Lay::LDK, S);
#pragma unroll
        for (int mt = 0; mt < MC; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                E[mt][r] = to_f32(sU[(16 * mt + 4 * g + r) * Lay::LDU + 16 * wv + l16]) - E[mt][r];

        // O = Q S + A E
        f32x4 O[MC];
#pragma unroll
        for (int mt = 0; mt < MC; ++mt) O[mt] = zero4();
        mm_acc_b<T, MC, MK, false, false>(O, sQ, Lay::LDK, S);
        mm_acc_b<T, MC, MC, true, false>(O, sA, Lay::LDC, E);

        // S += K^T E   (A = K^T: element (i = d_k row, k = token) at sK[k*LDK + i])
        mm_acc_b<T, MK, MC, false, true>(S, sK, Lay::LDK, E);

        T *op = o + tok0 * DV;
#pragma unroll
        for (int mt = 0; mt < MC; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * mt + 4 * g + r;
                if (row < valid) op[(long)row * DV + col] = from_f32<T>(O[mt][r]);
            }
    }

#pragma unroll
    for (int mk = 0; mk < MK; ++mk)
#pragma unroll
        for (int r = 0; r < 4; ++r) SL[sbase + (16 * mk + 4 * g + r) * DV + col] = S[mk][r];
}

template <typename T, int DK, int DV, int C, int NW>
hipError_t launch_scan(const void *q, const void *k, const void *w, const void *u, const void *aqk,
                       const float *S0, void *o, float *SL, int BH, int L, hipStream_t st)
{
    using Lay = ScanLayout<T, DK, DV, C, NW>;
    constexpr int NTILE = DV / Lay::TV;
    const int nchunks = (L + C - 1) / C;
    if (BH == 0) return hipSuccess;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&scan_kernel<T, DK, DV, C, NW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((scan_kernel<T, DK, DV, C, NW>), dim3((unsigned)(BH * NTILE)),
                       dim3(64 * NW), Lay::bytes, st, static_cast<const T *>(q),
                       static_cast<const T *>(k), static_cast<const T *>(w),
                       static_cast<const T *>(u), static_cast<const T *>(aqk), S0,
                       static_cast<T *>(o), SL, L, nchunks);
    return hipGetLastError();
}

// Waves per workgroup (1, 2 or 4; an explicit nw > 0 caps it).
template <typename T, int DK, int DV, int C>
hipError_t launch_scan_auto(const void *q, const void *k, const void *w, const void *u,
                            const void *aqk, const float *S0, void *o, float *SL, int BH, int L,
                            int nw, hipStream_t st)
{
    // Every wave owns 16 columns whatever NW is (the number of waves, hence of
    // busy SIMDs, is BH * DV / 16); wider tiles share each chunk's loads
    // between more waves.
    if (nw <= 0) nw = DV >= 64 ? 4 : DV >= 32 ? 2 : 1;
    if (nw >= 4 && DV >= 64)
        return launch_scan<T, DK, DV, C, 4>(q, k, w, u, aqk, S0, o, SL, BH, L, st);
    if (nw >= 2 && DV >= 32)
        return launch_scan<T, DK, DV, C, 2>(q, k, w, u, aqk, S0, o, SL, BH, L, st);
    return launch_scan<T, DK, DV, C, 1>(q, k, w, u, aqk, S0, o, SL, BH, L, st);
}

hipError_t dispatch_scan(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                         const void *w, const void *u, const void *aqk, const float *S0, void *o,
                         float *SL, int BH, int L, int nw, hipStream_t st)
{
#define CASE(DKV, DVV, CC)                                                                      \
    if (dk == DKV && dv == DVV && chunk == CC)                                                  \
        return bf16 ? launch_scan_auto<__bf16, DKV, DVV, CC>(q, k, w, u, aqk, S0, o, SL, BH, L, \
                                                             nw, st)                            \
                    : launch_scan_auto<float, DKV, DVV, CC>(q, k, w, u, aqk, S0, o, SL, BH, L,  \
                                                            nw, st);
    EFLA_SHAPE_CASES(CASE)
#undef CASE
    return hipErrorInvalidValue;
}

}  // namespace efla
