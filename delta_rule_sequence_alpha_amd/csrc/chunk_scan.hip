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
//
// Segment scan over L.  A chunk maps its entry state affinely, S -> P S + R
// with P = I - K^T W and R = K^T U, and these maps compose, so a sequence
// split into G chunk-aligned segments is scanned in three launches:
//   SUMMARY: every (sequence, segment) in parallel forms its segment's map --
//            R, the state reached from S = 0 (the usual columns), and P, the
//            state reached from S = I with U = 0 (d_k extra columns);
//   combine: S_in(0) = S0, S_in(g) = P_{g-1} S_in(g-1) + R_{g-1};
//   REPLAY:  every (sequence, segment) in parallel from S_in(g), writing o,
//            and the last segment S_L.
#include "efla_device.h"
#include "efla_launch.h"

namespace efla {

enum ScanMode { SCAN_WHOLE = 0, SCAN_SUMMARY = 1, SCAN_REPLAY = 2 };

struct SegArgs {
    int mode;          // ScanMode
    int G;             // segments per sequence (1 for SCAN_WHOLE)
    int seg_chunks;    // chunks per segment (the last one may be shorter)
    float *R;          // SUMMARY: [BH, G, DK, DV]
    float *P;          // SUMMARY: [BH, G, DK, DK]
    const float *Sin;  // REPLAY: [BH, G, DK, DV]
    void *states;      // WHOLE, optional: the entry state of every chunk [BH, nchunks, DK, DV],
                       // stored in the input dtype
    // Packed sequences (cu != NULL): BH = N * H with bh = seq * H + h; head
    // h's L tokens hold the N sequences back to back, sequence seq at
    // [cu[seq], cu[seq+1]), and A is stored by token ([H, L, C], valid rows
    // only).  Each sequence is split into G segments of ceil(chunks / G)
    // chunks (seg_chunks is not used); a segment with no chunk maps its
    // entry state to itself.
    const int *cu = nullptr;
    int H = 1;
};

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

// The scan of workgroup `bid` of `nblocks` (a kernel body, so that a launch
// can also host another scan's workgroups).
template <typename T, int DK, int DV, int C, int NW>
__device__ __forceinline__ void scan_body(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ w,
    const T *__restrict__ u, const T *__restrict__ aqk, const float *__restrict__ S0,
    T *__restrict__ o, float *__restrict__ SL, int L, int nchunks, SegArgs sg, int bid,
    int nblocks)
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

    // workgroup -> (sequence bh, segment gs, column tile); SUMMARY adds the
    // DK / TV tiles of P after the NTILE tiles of R, and runs segments
    // 0 .. G-2 only (the combine never reads the last segment's map)
    const int ntiles = NTILE + (sg.mode == SCAN_SUMMARY ? DK / TV : 0);
    const int Gl = sg.mode == SCAN_SUMMARY ? sg.G - 1 : sg.G;   // segments launched
    int bhs, tile;
    xcd_map_rr(bid, nblocks, ntiles, bhs, tile);
    const int bh = bhs / Gl, gs = bhs - bh * Gl;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
    const bool ptile = tile >= NTILE;                 // a column of P (U = 0, from S = I)
    const int utile = ptile ? 0 : tile;               // U columns read (ignored for P)
    const int col = (ptile ? tile - NTILE : tile) * TV + 16 * wv + l16;   // this lane's column
    // this sequence's tokens and chunks
    long tokb = (long)bh * L;
    int Ls = L, seg_chunks = sg.seg_chunks;
    if (sg.cu) {
        const int seq = bh / sg.H, h = bh - seq * sg.H;
        const int t0 = packed_begin(sg.cu, seq, L);
        tokb = (long)h * L + t0;
        Ls = packed_end(sg.cu, seq, L) - t0;
        nchunks = (Ls + C - 1) / C;
        seg_chunks = sg.G > 1 ? (nchunks + sg.G - 1) / sg.G : nchunks;
    }
    const int c_begin = gs * seg_chunks, c_end = min(nchunks, c_begin + seg_chunks);
    // chunk c's A block: per chunk, or (packed) by token
    auto a_at = [&](int c) {
        return sg.cu ? aqk + (tokb + (long)c * C) * C : aqk + ((long)bh * nchunks + c) * C * C;
    };

    f32x4 S[MK];
    const long sbase = (long)bh * DK * DV;
    const long segbase = ((long)bh * sg.G + gs) * DK * DV;
    if (sg.mode == SCAN_REPLAY) {
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int r = 0; r < 4; ++r) S[mk][r] = sg.Sin[segbase + (16 * mk + 4 * g + r) * DV + col];
    } else if (sg.mode == SCAN_SUMMARY) {
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int r = 0; r < 4; ++r) S[mk][r] = (ptile && 16 * mk + 4 * g + r == col) ? 1.f : 0.f;
    } else if (S0) {   // one branch around all the loads, so they are in flight together
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
    // (with no o to write, Q and A are not needed)
    const bool want_o = sg.mode != SCAN_SUMMARY && o;
    auto load_all = [&](int cn) {
        cn = min(cn, c_end - 1);
        const long t0 = tokb + (long)cn * C;
        const int vn = min(C, Ls - cn * C);
        rW.load(w + t0 * DK, DK, vn);
        rK.load(k + t0 * DK, DK, vn);
        if (!ptile) rU.load(u + t0 * DV + utile * TV, DV, vn);   // (a map's matrix: U = 0)
        if (want_o) {
            rQ.load(q + t0 * DK, DK, vn);
            rA.load(a_at(cn), C, sg.cu ? vn : C);
        }
    };
    if constexpr (PREFETCH) {
        if (c_begin < c_end) load_all(c_begin);
    }

    for (int c = c_begin; c < c_end; ++c) {
        const long tok0 = tokb + (long)c * C;
        const int valid = min(C, Ls - c * C);
        __syncthreads();   // the previous chunk is done with LDS (and this chunk's loads have landed)
        if constexpr (PREFETCH) {
            rW.store(sW, Lay::LDK, valid);
            rK.store(sK, Lay::LDK, valid);
            if (!ptile) rU.store(sU, Lay::LDU, valid);
            if (want_o) {
                rQ.store(sQ, Lay::LDK, valid);
                rA.store(sA, Lay::LDC, sg.cu ? valid : C);
            }
        } else {
            RW t;
            t.load(w + tok0 * DK, DK, valid);
            t.store(sW, Lay::LDK, valid);
            t.load(k + tok0 * DK, DK, valid);
            t.store(sK, Lay::LDK, valid);
            if (!ptile) {
                rU.load(u + tok0 * DV + utile * TV, DV, valid);
                rU.store(sU, Lay::LDU, valid);
            }
            if (want_o) {
                t.load(q + tok0 * DK, DK, valid);
                t.store(sQ, Lay::LDK, valid);
                const int arows = sg.cu ? valid : C;
                rA.load(a_at(c), C, arows);
                rA.store(sA, Lay::LDC, arows);
            }
        }
        __syncthreads();
        // the next chunk's loads fly while this one is computed (a workgroup
        // barrier waits for every outstanding load, so they are issued after it)
        if constexpr (PREFETCH) load_all(c + 1);

        if (sg.states) {
            T *st = static_cast<T *>(sg.states) + ((long)bh * nchunks + c) * DK * DV;
#pragma unroll
            for (int mk = 0; mk < MK; ++mk)
#pragma unroll
                for (int r = 0; r < 4; ++r) st[(16 * mk + 4 * g + r) * DV + col] = from_f32<T>(S[mk][r]);
        }

        // E = U - W S
        f32x4 E[MC];
#pragma unroll
        for (int mt = 0; mt < MC; ++mt) E[mt] = zero4();
        mm_acc_b<T, MC, MK, false, false>(E, sW, Lay::LDK, S);
#pragma unroll
        for (int mt = 0; mt < MC; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                E[mt][r] = (ptile ? 0.f : to_f32(sU[(16 * mt + 4 * g + r) * Lay::LDU + 16 * wv + l16])) -
                           E[mt][r];

        if (want_o) {   // a segment's map needs no output
            // O = Q S + A E
            f32x4 O[MC];
#pragma unroll
            for (int mt = 0; mt < MC; ++mt) O[mt] = zero4();
            mm_acc_b<T, MC, MK, false, false>(O, sQ, Lay::LDK, S);
            mm_acc_b<T, MC, MC, true, false>(O, sA, Lay::LDC, E);
            T *op = o + tok0 * DV;
#pragma unroll
            for (int mt = 0; mt < MC; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * mt + 4 * g + r;
                    if (row < valid) op[(long)row * DV + col] = from_f32<T>(O[mt][r]);
                }
        }

        // S += K^T E   (A = K^T: element (i = d_k row, k = token) at sK[k*LDK + i])
        mm_acc_b<T, MK, MC, false, true>(S, sK, Lay::LDK, E);
    }

    if (sg.mode != SCAN_SUMMARY && !SL) return;
    float *dst = SL + sbase;
    int ld = DV;
    if (sg.mode == SCAN_SUMMARY) {
        dst = ptile ? sg.P + ((long)bh * sg.G + gs) * DK * DK : sg.R + segbase;
        ld = ptile ? DK : DV;
    } else if (sg.mode == SCAN_REPLAY && gs != sg.G - 1) {
        return;   // only the last segment's final state is the sequence's
    }
#pragma unroll
    for (int mk = 0; mk < MK; ++mk)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * mk + 4 * g + r) * ld + col] = S[mk][r];
}

template <typename T, int DK, int DV, int C, int NW>
__global__ __launch_bounds__(64 * NW) void scan_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ w,
    const T *__restrict__ u, const T *__restrict__ aqk, const float *__restrict__ S0,
    T *__restrict__ o, float *__restrict__ SL, int L, int nchunks, SegArgs sg)
{
    scan_body<T, DK, DV, C, NW>(q, k, w, u, aqk, S0, o, SL, L, nchunks, sg, blockIdx.x, gridDim.x);
}

// S_in(0) = S0 (or 0); S_in(g) = P_{g-1} S_in(g-1) + R_{g-1} for g = 1 .. G-1.
// One workgroup of four waves per (sequence, 16 columns).  The 16 columns of
// S_in(g-1) stay in LDS; P_{g-1} is staged in LDS from registers, into which
// P_g (and the R tiles of step g) are loaded meanwhile; each wave forms
// DK / 64 row tiles of the product on fp32 MFMA.
template <int DK, int DV>
struct CombineLayout {
    static constexpr int LDP = DK + 4;    // P rows: 16-byte aligned, conflict-free row reads
    static constexpr int LDS_ = 17;       // the state's 16 columns, read by rows 4 apart
    static constexpr size_t offP = 0;
    static constexpr size_t offS = offP + sizeof(float) * DK * LDP;
    static constexpr size_t bytes = offS + sizeof(float) * DK * LDS_;
};

template <int DK, int DV>
__global__ __launch_bounds__(256) void seg_combine_kernel(const float *__restrict__ S0,
                                                          const float *__restrict__ P,
                                                          const float *__restrict__ R,
                                                          float *__restrict__ Sin, int G)
{
    using Lay = CombineLayout<DK, DV>;
    constexpr int NCB = DV / 16, MK = DK / 16, TPW = (MK + 3) / 4;   // row tiles per wave
    extern __shared__ __align__(16) char smem[];
    float *sP = reinterpret_cast<float *>(smem + Lay::offP);
    float *sS = reinterpret_cast<float *>(smem + Lay::offS);
    const int bh = blockIdx.x / NCB, cb = blockIdx.x - bh * NCB;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6, l16 = lane & 15, g = lane >> 4;
    for (int e = t; e < DK * 16; e += 256) {
        const int i = e >> 4, jj = e & 15;
        const float x = S0 ? S0[((long)bh * DK + i) * DV + cb * 16 + jj] : 0.f;
        sS[i * Lay::LDS_ + jj] = x;
        Sin[(((long)bh * G) * DK + i) * DV + cb * 16 + jj] = x;
    }
    TileRegs<float, DK, DK, 256> rP;
    f32x4 rR[TPW];
    auto load_step = [&](int gs) {   // P_{gs-1} and this wave's tiles of R_{gs-1}
        rP.load(P + ((long)bh * G + gs - 1) * DK * DK, DK, DK);
        const float *Rg = R + ((long)bh * G + gs - 1) * DK * DV + cb * 16 + l16;
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int mt = wv + 4 * u;
            if (mt < MK)
#pragma unroll
                for (int r = 0; r < 4; ++r) rR[u][r] = Rg[(long)(16 * mt + 4 * g + r) * DV];
        }
    };
    if (G > 1) load_step(1);
    for (int gs = 1; gs < G; ++gs) {
        rP.store(sP, Lay::LDP, DK);
        f32x4 acc[TPW];
#pragma unroll
        for (int u = 0; u < TPW; ++u) acc[u] = rR[u];
        __syncthreads();   // P_{gs-1} and S_in(gs-1) in LDS
        if (gs + 1 < G) load_step(gs + 1);
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int mt = wv + 4 * u;
            if (mt < MK)
                acc[u] = mm_lds<float, DK, false, true>(acc[u], sP, Lay::LDP, 16 * mt, sS,
                                                        Lay::LDS_, 0);
        }
        __syncthreads();   // every read of S_in(gs-1) and P_{gs-1} is done
        float *dst = Sin + (((long)bh * G + gs) * DK) * DV + cb * 16 + l16;
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int mt = wv + 4 * u;
            if (mt < MK)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * mt + 4 * g + r;
                    sS[row * Lay::LDS_ + l16] = acc[u][r];
                    dst[(long)row * DV] = acc[u][r];
                }
        }
    }
}

template <int DK, int DV>
hipError_t launch_combine(const float *S0, const float *P, const float *R, float *Sin, int BH,
                          int G, hipStream_t st)
{
    using Lay = CombineLayout<DK, DV>;
    const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&seg_combine_kernel<DK, DV>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((seg_combine_kernel<DK, DV>), dim3((unsigned)(BH * (DV / 16))), dim3(256),
                       Lay::bytes, st, S0, P, R, Sin, G);
    return hipGetLastError();
}

template <typename T, int DK, int DV, int C, int NW>
hipError_t launch_scan(const void *q, const void *k, const void *w, const void *u, const void *aqk,
                       const float *S0, void *o, float *SL, int BH, int L, SegArgs sg,
                       hipStream_t st)
{
    using Lay = ScanLayout<T, DK, DV, C, NW>;
    const int ntiles = DV / Lay::TV + (sg.mode == SCAN_SUMMARY ? DK / Lay::TV : 0);
    const int nchunks = (L + C - 1) / C;
    const int Gl = sg.mode == SCAN_SUMMARY ? sg.G - 1 : sg.G;   // see scan_body
    if (BH == 0 || Gl <= 0) return hipSuccess;
    const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&scan_kernel<T, DK, DV, C, NW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((scan_kernel<T, DK, DV, C, NW>), dim3((unsigned)(BH * Gl * ntiles)),
                       dim3(64 * NW), Lay::bytes, st, static_cast<const T *>(q),
                       static_cast<const T *>(k), static_cast<const T *>(w),
                       static_cast<const T *>(u), static_cast<const T *>(aqk), S0,
                       static_cast<T *>(o), SL, L, nchunks, sg);
    return hipGetLastError();
}

// Waves per workgroup (1, 2 or 4; an explicit nw > 0 caps it).  The
// segment summary also tiles the d_k columns of P, so there the tile must
// divide d_k too.
template <typename T, int DK, int DV, int C>
hipError_t launch_scan_auto(const void *q, const void *k, const void *w, const void *u,
                            const void *aqk, const float *S0, void *o, float *SL, int BH, int L,
                            int nw, SegArgs sg, hipStream_t st)
{
    // Every wave owns 16 columns whatever NW is (the number of waves, hence of
    // busy SIMDs, is BH * DV / 16); wider tiles share each chunk's loads
    // between more waves.  By default 4 waves; the fp32 segment passes at
    // d_k = d_v = 128 take 8 (128 columns): their 153 KB workgroup is alone
    // on its CU either way, and 8 waves give each SIMD two to alternate
    // between while one waits on LDS.
    constexpr int DMIN = DK < DV ? DK : DV;
    const int wmax = sg.mode == SCAN_SUMMARY ? DMIN : DV;
    constexpr bool WIDE = !is_bf16<T> && DMIN >= 128;
    if (nw <= 0) nw = (WIDE && sg.mode != SCAN_WHOLE) ? 8 : 4;
    if constexpr (WIDE) {
        if (nw >= 8 && wmax >= 128)
            return launch_scan<T, DK, DV, C, 8>(q, k, w, u, aqk, S0, o, SL, BH, L, sg, st);
    }
    if (nw >= 4 && wmax >= 64)
        return launch_scan<T, DK, DV, C, 4>(q, k, w, u, aqk, S0, o, SL, BH, L, sg, st);
    if (nw >= 2 && wmax >= 32)
        return launch_scan<T, DK, DV, C, 2>(q, k, w, u, aqk, S0, o, SL, BH, L, sg, st);
    return launch_scan<T, DK, DV, C, 1>(q, k, w, u, aqk, S0, o, SL, BH, L, sg, st);
}

template <typename T, int DK, int DV, int C>
hipError_t launch_scan_segmented(const void *q, const void *k, const void *w, const void *u,
                                 const void *aqk, const float *S0, void *o, float *SL, int BH,
                                 int L, int G, int seg_chunks, float *R, float *P, float *Sin,
                                 int nw, const int *cu, int H, hipStream_t st)
{
    if (BH == 0) return hipSuccess;
    SegArgs sum{SCAN_SUMMARY, G, seg_chunks, R, P, nullptr, nullptr, cu, H};
    hipError_t e = launch_scan_auto<T, DK, DV, C>(q, k, w, u, aqk, nullptr, o, SL, BH, L, nw, sum, st);
    if (e != hipSuccess) return e;
    e = launch_combine<DK, DV>(S0, P, R, Sin, BH, G, st);
    if (e != hipSuccess) return e;
    SegArgs rep{SCAN_REPLAY, G, seg_chunks, nullptr, nullptr, Sin, nullptr, cu, H};
    return launch_scan_auto<T, DK, DV, C>(q, k, w, u, aqk, nullptr, o, SL, BH, L, nw, rep, st);
}

// ---------------------------------------------------------------------------
// Reverse state scan of the backward pass.  The chunk map above,
//   E = U - W S_in,  O = Q S_in + A E,  S_out = S_in + K^T E,
// sends the gradient dS_out = dLoss/dS_out back through the chunk as
//   dE    = A^T dO + K dS_out                   (the chunk's dLoss/dE)
//   dS_in = dS_out + Q^T dO - W^T dE            (W^T dE = K^T T^T dE)
// which, like the forward, never mixes the d_v columns: a workgroup owns a
// (sequence, column tile), walks the chunks from last to first with dS in
// MFMA accumulators, and stores every chunk's dS_out and dE (in the input
// dtype: bf16 inputs' products round them to bf16 anyway) for the
// per-chunk gradient kernel.  dS0 receives dLoss/dS0.
//
// Segments, as in the forward: the chunk sends dS_out to
// dS_in = (I - W^T K) dS_out + (Q^T - W^T A^T) dO, an affine map whose
// matrix is the transpose of the forward one, so a sequence split into G
// segments is scanned backwards in three launches: SUMMARY forms each
// segment's map (R from dS = 0, the matrix from dS = I with dO = 0), the
// combine pass runs the maps from the last segment to the first (stored in
// reverse segment order, so the forward combine kernel serves), and REPLAY
// walks every segment from its true end gradient, storing dS_out and dE.
template <typename T, int DK, int DV, int C, int NW>
__device__ __forceinline__ void rscan_body(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ w,
    const T *__restrict__ aqk, const T *__restrict__ dout, const float *__restrict__ dSL,
    T *__restrict__ dSout, T *__restrict__ dE, float *__restrict__ dS0, int L, int nchunks,
    SegArgs sg, int bid, int nblocks)
{
    using Lay = ScanLayout<T, DK, DV, C, NW>;
    constexpr int TV = Lay::TV, NTILE = DV / TV, MC = C / 16, MK = DK / 16;
    constexpr int NT = 64 * NW;
    extern __shared__ __align__(16) char smem[];
    T *sW = reinterpret_cast<T *>(smem + Lay::offW);
    T *sQ = reinterpret_cast<T *>(smem + Lay::offQ);
    T *sK = reinterpret_cast<T *>(smem + Lay::offK);
    T *sA = reinterpret_cast<T *>(smem + Lay::offA);
    T *sO = reinterpret_cast<T *>(smem + Lay::offU);   // the dO column tile

    const bool summary = sg.mode == SCAN_SUMMARY;
    const int ntiles = NTILE + (summary ? DK / TV : 0);
    int bhs, tile;
    xcd_map(bid, nblocks, ntiles, bhs, tile);
    const int bh = bhs / sg.G, gs = bhs - bh * sg.G;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
    const bool ptile = tile >= NTILE;                 // a column of the map's matrix (dO = 0, from I)
    const int utile = ptile ? 0 : tile;
    const int col = (ptile ? tile - NTILE : tile) * TV + 16 * wv + l16;
    const long sbase = (long)bh * DK * DV;
    const int c_begin = gs * sg.seg_chunks, c_end = min(nchunks, c_begin + sg.seg_chunks);
    const long segbase = ((long)bh * sg.G + (sg.G - 1 - gs)) * DK * DV;   // reverse order

    f32x4 dS[MK];
    if (sg.mode == SCAN_REPLAY) {
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int r = 0; r < 4; ++r) dS[mk][r] = sg.Sin[segbase + (16 * mk + 4 * g + r) * DV + col];
    } else if (summary) {
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int r = 0; r < 4; ++r) dS[mk][r] = (ptile && 16 * mk + 4 * g + r == col) ? 1.f : 0.f;
    } else if (dSL) {
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int r = 0; r < 4; ++r) dS[mk][r] = dSL[sbase + (16 * mk + 4 * g + r) * DV + col];
    } else {
#pragma unroll
        for (int mk = 0; mk < MK; ++mk) dS[mk] = zero4();
    }

    // As in the forward scan: the previous chunk's tiles are loaded while
    // this one is computed, unless they would not fit in registers.
    using RW = TileRegs<T, C, DK, NT>;
    using RU = TileRegs<T, C, TV, NT>;
    using RA = TileRegs<T, C, C, NT>;
    constexpr bool PREFETCH = 3 * RW::PER + RU::PER + RA::PER <= 40;
    RW rW, rQ, rK;
    RU rO;
    RA rA;
    auto load_all = [&](int cn) {   // chunk cn's tiles (cn < c_begin re-loads c_begin, never stored)
        cn = max(cn, c_begin);
        const long t0 = (long)bh * L + (long)cn * C;
        const int vn = min(C, L - cn * C);
        rW.load(w + t0 * DK, DK, vn);
        rQ.load(q + t0 * DK, DK, vn);
        rK.load(k + t0 * DK, DK, vn);
        rO.load(dout + t0 * DV + utile * TV, DV, vn);
        rA.load(aqk + ((long)bh * nchunks + cn) * C * C, C, C);
    };
    if constexpr (PREFETCH) {
        if (c_end > c_begin) load_all(c_end - 1);
    }

    for (int c = c_end - 1; c >= c_begin; --c) {
        const int valid = min(C, L - c * C);
        const long tok0 = (long)bh * L + (long)c * C;
        __syncthreads();   // the previous chunk is done with LDS
        if constexpr (PREFETCH) {
            rW.store(sW, Lay::LDK, valid);
            rQ.store(sQ, Lay::LDK, valid);
            rK.store(sK, Lay::LDK, valid);
            rO.store(sO, Lay::LDU, valid);
            rA.store(sA, Lay::LDC, C);
        } else {
            RW t;
            t.load(w + tok0 * DK, DK, valid);
            t.store(sW, Lay::LDK, valid);
            t.load(q + tok0 * DK, DK, valid);
            t.store(sQ, Lay::LDK, valid);
            t.load(k + tok0 * DK, DK, valid);
            t.store(sK, Lay::LDK, valid);
            rO.load(dout + tok0 * DV + utile * TV, DV, valid);
            rO.store(sO, Lay::LDU, valid);
            rA.load(aqk + ((long)bh * nchunks + c) * C * C, C, C);
            rA.store(sA, Lay::LDC, C);
        }
        __syncthreads();
        if constexpr (PREFETCH) load_all(c - 1);   // in flight during this chunk

        if (!summary) {   // a segment's map stores nothing per chunk
            T *so = dSout + ((long)bh * nchunks + c) * DK * DV;
#pragma unroll
            for (int mk = 0; mk < MK; ++mk)
#pragma unroll
                for (int r = 0; r < 4; ++r) so[(16 * mk + 4 * g + r) * DV + col] = from_f32<T>(dS[mk][r]);
        }

        f32x4 dO[MC], dEc[MC];
#pragma unroll
        for (int mt = 0; mt < MC; ++mt) {
            dEc[mt] = zero4();
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dO[mt][r] = ptile ? 0.f : to_f32(sO[(16 * mt + 4 * g + r) * Lay::LDU + 16 * wv + l16]);
        }
        // dE = K dS_out + A^T dO   (A^T: element (i, m) = A[m][i]; A is zero above its diagonal)
        mm_acc_b<T, MC, MK, false, false>(dEc, sK, Lay::LDK, dS);
        mm_acc_b<T, MC, MC, false, true>(dEc, sA, Lay::LDC, dO);
        if (!summary) {
            T *de = dE + ((long)bh * nchunks * C + (long)c * C) * DV;
#pragma unroll
            for (int mt = 0; mt < MC; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) de[(16 * mt + 4 * g + r) * DV + col] = from_f32<T>(dEc[mt][r]);
        }

        // dS <- dS + Q^T dO - W^T dE
        mm_acc_b<T, MK, MC, false, true>(dS, sQ, Lay::LDK, dO);
#pragma unroll
        for (int mt = 0; mt < MC; ++mt) dEc[mt] = -dEc[mt];
        mm_acc_b<T, MK, MC, false, true>(dS, sW, Lay::LDK, dEc);
    }

    float *dst = dS0 ? dS0 + sbase : nullptr;
    int ld = DV;
    if (summary) {
        dst = ptile ? sg.P + ((long)bh * sg.G + (sg.G - 1 - gs)) * DK * DK : sg.R + segbase;
        ld = ptile ? DK : DV;
    } else if (gs != 0) {
        return;   // only the first segment's final gradient is dLoss/dS0
    }
    if (dst) {
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(16 * mk + 4 * g + r) * ld + col] = dS[mk][r];
    }
}

template <typename T, int DK, int DV, int C, int NW>
__global__ __launch_bounds__(64 * NW) void rscan_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ w,
    const T *__restrict__ aqk, const T *__restrict__ dout, const float *__restrict__ dSL,
    T *__restrict__ dSout, T *__restrict__ dE, float *__restrict__ dS0, int L, int nchunks,
    SegArgs sg)
{
    rscan_body<T, DK, DV, C, NW>(q, k, w, aqk, dout, dSL, dSout, dE, dS0, L, nchunks, sg,
                                 blockIdx.x, gridDim.x);
}

// The backward's two scans in one launch: they are independent (the reverse
// scan needs no chunk state), and each is latency-bound on its own chain of
// chunks, so workgroups of both sharing the CUs hide each other's waits.
// Workgroups [0, nfwd) run the state scan, the rest the reverse scan.
template <typename T, int DK, int DV, int C, int NW>
__global__ __launch_bounds__(64 * NW) void scan_pair_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ w,
    const T *__restrict__ u, const T *__restrict__ aqk, const float *__restrict__ S0,
    void *states, const T *__restrict__ dout, const float *__restrict__ dSL,
    T *__restrict__ dSout, T *__restrict__ dE, float *__restrict__ dS0, int L, int nchunks,
    int nfwd)
{
    const int b = blockIdx.x;
    if (b < nfwd) {
        const SegArgs whole{SCAN_WHOLE, 1, 1 << 30, nullptr, nullptr, nullptr, states};
        scan_body<T, DK, DV, C, NW>(q, k, w, u, aqk, S0, nullptr, nullptr, L, nchunks, whole, b,
                                    nfwd);
    } else {
        const SegArgs whole{SCAN_WHOLE, 1, 1 << 30, nullptr, nullptr, nullptr, nullptr};
        rscan_body<T, DK, DV, C, NW>(q, k, w, aqk, dout, dSL, dSout, dE, dS0, L, nchunks, whole,
                                     b - nfwd, (int)gridDim.x - nfwd);
    }
}

template <typename T, int DK, int DV, int C, int NW>
hipError_t launch_rscan_nw(const void *q, const void *k, const void *w, const void *aqk,
                           const void *dout, const float *dSL, void *dSout, void *dE, float *dS0,
                           int BH, int L, SegArgs sg, hipStream_t st)
{
    using Lay = ScanLayout<T, DK, DV, C, NW>;
    const int ntiles = DV / Lay::TV + (sg.mode == SCAN_SUMMARY ? DK / Lay::TV : 0);
    const int nchunks = (L + C - 1) / C;
    if (BH == 0) return hipSuccess;
    const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&rscan_kernel<T, DK, DV, C, NW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((rscan_kernel<T, DK, DV, C, NW>), dim3((unsigned)(BH * sg.G * ntiles)),
                       dim3(64 * NW), Lay::bytes, st, static_cast<const T *>(q),
                       static_cast<const T *>(k), static_cast<const T *>(w),
                       static_cast<const T *>(aqk), static_cast<const T *>(dout), dSL,
                       static_cast<T *>(dSout), static_cast<T *>(dE),
                       dS0, L, nchunks, sg);
    return hipGetLastError();
}

// Waves per workgroup (each owns 16 columns): 4 unless nw > 0 caps it; the
// segment summary also tiles the d_k columns of the map's matrix.
template <typename T, int DK, int DV, int C>
hipError_t launch_rscan_mode(const void *q, const void *k, const void *w, const void *aqk,
                             const void *dout, const float *dSL, void *dSout, void *dE,
                             float *dS0, int BH, int L, int nw, SegArgs sg, hipStream_t st)
{
    constexpr int DMIN = DK < DV ? DK : DV;
    const int wmax = sg.mode == SCAN_SUMMARY ? DMIN : DV;
    if (nw <= 0) nw = 4;
    if (nw >= 4 && wmax >= 64)
        return launch_rscan_nw<T, DK, DV, C, 4>(q, k, w, aqk, dout, dSL, dSout, dE, dS0, BH, L, sg, st);
    if (nw >= 2 && wmax >= 32)
        return launch_rscan_nw<T, DK, DV, C, 2>(q, k, w, aqk, dout, dSL, dSout, dE, dS0, BH, L, sg, st);
    return launch_rscan_nw<T, DK, DV, C, 1>(q, k, w, aqk, dout, dSL, dSout, dE, dS0, BH, L, sg, st);
}

// G == 1: one walk over each sequence.  G > 1: segment maps (R [BH,G,dk,dv],
// P [BH,G,dk,dk]), their composition from dS_L into each segment's end
// gradient (Sin [BH,G,dk,dv]), then every segment replayed in parallel; all
// three in reverse segment order.
template <typename T, int DK, int DV, int C>
hipError_t launch_rscan(const void *q, const void *k, const void *w, const void *aqk,
                        const void *dout, const float *dSL, void *dSout, void *dE, float *dS0,
                        int BH, int L, int nw, int G, int seg_chunks, float *R, float *P,
                        float *Sin, hipStream_t st)
{
    if (G <= 1) {
        const SegArgs whole{SCAN_WHOLE, 1, 1 << 30, nullptr, nullptr, nullptr, nullptr};
        return launch_rscan_mode<T, DK, DV, C>(q, k, w, aqk, dout, dSL, dSout, dE, dS0, BH, L, nw,
                                               whole, st);
    }
    if (BH == 0) return hipSuccess;
    const SegArgs sum{SCAN_SUMMARY, G, seg_chunks, R, P, nullptr, nullptr};
    hipError_t e = launch_rscan_mode<T, DK, DV, C>(q, k, w, aqk, dout, nullptr, dSout, dE, nullptr,
                                                   BH, L, nw, sum, st);
    if (e != hipSuccess) return e;
    e = launch_combine<DK, DV>(dSL, P, R, Sin, BH, G, st);
    if (e != hipSuccess) return e;
    const SegArgs rep{SCAN_REPLAY, G, seg_chunks, nullptr, nullptr, Sin, nullptr};
    return launch_rscan_mode<T, DK, DV, C>(q, k, w, aqk, dout, nullptr, dSout, dE, dS0, BH, L, nw,
                                           rep, st);
}

hipError_t dispatch_rscan(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                          const void *w, const void *aqk, const void *dout, const float *dSL,
                          void *dSout, void *dE, float *dS0, int BH, int L, int nw, int G,
                          int seg_chunks, float *R, float *P, float *Sin, hipStream_t st)
{
#define CASE(DKV, DVV, CC)                                                                      \
    if (dk == DKV && dv == DVV && chunk == CC)                                                  \
        return bf16 ? launch_rscan<__bf16, DKV, DVV, CC>(q, k, w, aqk, dout, dSL, dSout, dE,    \
                                                         dS0, BH, L, nw, G, seg_chunks, R, P,   \
                                                         Sin, st)                               \
                    : launch_rscan<float, DKV, DVV, CC>(q, k, w, aqk, dout, dSL, dSout, dE,     \
                                                        dS0, BH, L, nw, G, seg_chunks, R, P,    \
                                                        Sin, st);
    EFLA_SHAPE_CASES(CASE)
#undef CASE
    return hipErrorInvalidValue;
}

hipError_t dispatch_scan_states(bool bf16, int dk, int dv, int chunk, const void *q,
                                const void *k, const void *w, const void *u, const void *aqk,
                                const float *S0, void *states, int BH, int L, int nw, int G,
                                int seg_chunks, float *R, float *P, float *Sin, hipStream_t st)
{
    if (G > 1) {   // segment maps, their composition, then the segments replayed storing states
        const SegArgs sum{SCAN_SUMMARY, G, seg_chunks, R, P, nullptr, nullptr};
        const SegArgs rep{SCAN_REPLAY, G, seg_chunks, nullptr, nullptr, Sin, states};
#define CASE(DKV, DVV, CC)                                                                      \
        if (dk == DKV && dv == DVV && chunk == CC) {                                            \
            hipError_t e = bf16 ? launch_scan_auto<__bf16, DKV, DVV, CC>(q, k, w, u, aqk, nullptr, \
                                      nullptr, nullptr, BH, L, nw, sum, st)                     \
                                : launch_scan_auto<float, DKV, DVV, CC>(q, k, w, u, aqk, nullptr, \
                                      nullptr, nullptr, BH, L, nw, sum, st);                    \
            if (e != hipSuccess) return e;                                                      \
            e = launch_combine<DKV, DVV>(S0, P, R, Sin, BH, G, st);                             \
            if (e != hipSuccess) return e;                                                      \
            return bf16 ? launch_scan_auto<__bf16, DKV, DVV, CC>(q, k, w, u, aqk, nullptr,      \
                                                                 nullptr, nullptr, BH, L, nw, rep, st) \
                        : launch_scan_auto<float, DKV, DVV, CC>(q, k, w, u, aqk, nullptr,       \
                                                                nullptr, nullptr, BH, L, nw, rep, st); \
        }
        EFLA_SHAPE_CASES(CASE)
#undef CASE
        return hipErrorInvalidValue;
    }
    const SegArgs whole{SCAN_WHOLE, 1, 1 << 30, nullptr, nullptr, nullptr, states};
#define CASE(DKV, DVV, CC)                                                                      \
    if (dk == DKV && dv == DVV && chunk == CC)                                                  \
        return bf16 ? launch_scan_auto<__bf16, DKV, DVV, CC>(q, k, w, u, aqk, S0, nullptr,      \
                                                             nullptr, BH, L, nw, whole, st)     \
                    : launch_scan_auto<float, DKV, DVV, CC>(q, k, w, u, aqk, S0, nullptr,       \
                                                            nullptr, BH, L, nw, whole, st);
    EFLA_SHAPE_CASES(CASE)
#undef CASE
    return hipErrorInvalidValue;
}

template <typename T, int DK, int DV, int C, int NW>
hipError_t launch_scan_pair_nw(const void *q, const void *k, const void *w, const void *u,
                               const void *aqk, const float *S0, void *states, const void *dout,
                               const float *dSL, void *dSout, void *dE, float *dS0, int BH, int L,
                               hipStream_t st)
{
    using Lay = ScanLayout<T, DK, DV, C, NW>;
    const int nchunks = (L + C - 1) / C;
    const int nfwd = BH * (DV / Lay::TV);
    if (BH == 0) return hipSuccess;
    const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&scan_pair_kernel<T, DK, DV, C, NW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((scan_pair_kernel<T, DK, DV, C, NW>), dim3((unsigned)(2 * nfwd)),
                       dim3(64 * NW), Lay::bytes, st, static_cast<const T *>(q),
                       static_cast<const T *>(k), static_cast<const T *>(w),
                       static_cast<const T *>(u), static_cast<const T *>(aqk), S0, states,
                       static_cast<const T *>(dout), dSL, static_cast<T *>(dSout),
                       static_cast<T *>(dE), dS0, L, nchunks, nfwd);
    return hipGetLastError();
}

template <typename T, int DK, int DV, int C>
hipError_t launch_scan_pair(const void *q, const void *k, const void *w, const void *u,
                            const void *aqk, const float *S0, void *states, const void *dout,
                            const float *dSL, void *dSout, void *dE, float *dS0, int BH, int L,
                            int nw, hipStream_t st)
{
    if (nw <= 0) nw = 4;
    if (nw >= 4 && DV >= 64)
        return launch_scan_pair_nw<T, DK, DV, C, 4>(q, k, w, u, aqk, S0, states, dout, dSL, dSout,
                                                     dE, dS0, BH, L, st);
    if (nw >= 2 && DV >= 32)
        return launch_scan_pair_nw<T, DK, DV, C, 2>(q, k, w, u, aqk, S0, states, dout, dSL, dSout,
                                                     dE, dS0, BH, L, st);
    return launch_scan_pair_nw<T, DK, DV, C, 1>(q, k, w, u, aqk, S0, states, dout, dSL, dSout, dE,
                                                 dS0, BH, L, st);
}

hipError_t dispatch_scan_pair(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                              const void *w, const void *u, const void *aqk, const float *S0,
                              void *states, const void *dout, const float *dSL, void *dSout,
                              void *dE, float *dS0, int BH, int L, int nw, hipStream_t st)
{
#define CASE(DKV, DVV, CC)                                                                      \
    if (dk == DKV && dv == DVV && chunk == CC)                                                  \
        return bf16 ? launch_scan_pair<__bf16, DKV, DVV, CC>(q, k, w, u, aqk, S0, states, dout, \
                                                             dSL, dSout, dE, dS0, BH, L, nw, st) \
                    : launch_scan_pair<float, DKV, DVV, CC>(q, k, w, u, aqk, S0, states, dout,  \
                                                            dSL, dSout, dE, dS0, BH, L, nw, st);
    EFLA_SHAPE_CASES(CASE)
#undef CASE
    return hipErrorInvalidValue;
}

hipError_t dispatch_scan(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                         const void *w, const void *u, const void *aqk, const float *S0, void *o,
                         float *SL, int BH, int L, int nw, hipStream_t st, const int *cu, int H)
{
    const SegArgs whole{SCAN_WHOLE, 1, 1 << 30, nullptr, nullptr, nullptr, nullptr, cu, H};
#define CASE(DKV, DVV, CC)                                                                      \
    if (dk == DKV && dv == DVV && chunk == CC)                                                  \
        return bf16 ? launch_scan_auto<__bf16, DKV, DVV, CC>(q, k, w, u, aqk, S0, o, SL, BH, L, \
                                                             nw, whole, st)                     \
                    : launch_scan_auto<float, DKV, DVV, CC>(q, k, w, u, aqk, S0, o, SL, BH, L,  \
                                                            nw, whole, st);
    EFLA_SHAPE_CASES(CASE)
#undef CASE
    return hipErrorInvalidValue;
}

hipError_t dispatch_scan_segmented(bool bf16, int dk, int dv, int chunk, const void *q,
                                   const void *k, const void *w, const void *u, const void *aqk,
                                   const float *S0, void *o, float *SL, int BH, int L, int G,
                                   int seg_chunks, float *R, float *P, float *Sin, int nw,
                                   hipStream_t st, const int *cu, int H)
{
#define CASE(DKV, DVV, CC)                                                                      \
    if (dk == DKV && dv == DVV && chunk == CC)                                                  \
        return bf16 ? launch_scan_segmented<__bf16, DKV, DVV, CC>(                              \
                          q, k, w, u, aqk, S0, o, SL, BH, L, G, seg_chunks, R, P, Sin, nw, cu,  \
                          H, st)                                                                \
                    : launch_scan_segmented<float, DKV, DVV, CC>(                               \
                          q, k, w, u, aqk, S0, o, SL, BH, L, G, seg_chunks, R, P, Sin, nw, cu,  \
                          H, st);
    EFLA_SHAPE_CASES(CASE)
#undef CASE
    return hipErrorInvalidValue;
}

}  // namespace efla
