// Fused chunkwise EFLA forward: coefficients, the chunk-local UT quantities and
// the inter-chunk state scan in one kernel, with no intermediate HBM traffic.
// ("Exact Flow Linear Attention: Exact Solution from Continuous-Time
// Dynamics", Technical Summary, Methodology 3: the exact-flow update keeps the
// delta rule's rank-1 form and hence its WY/UT chunkwise parallelism.)
//
// Per chunk of C tokens with entry state S, keys K, queries Q, values V and
// a = alpha, G = K K^T, D = diag(a):
//   (I + D strictly_lower(G)) E = D (V - K S)            (E: stacked e_r^T)
//   O = Q S + tril(Q K^T) E,   S <- S + K^T E.
// The triangular system is solved on 16-row blocks,
//   E_i = T_ii (X_i - sum_{m<i} G_im E_m),  X = V - K S,
//   T_ii = (I + D_i strictly_lower(G_ii))^{-1} D_i,
// with T_ii from forward substitution in fp32 (no division by alpha).
//
// Workgroup = (sequence, tile of TV = 16*NS state columns), NS + 2 waves:
//  * scan waves (0 .. NS-1): wave w keeps 16 columns x all d_k rows of S in
//    MFMA accumulators and runs only the S-dependent chain of each chunk:
//    K S, Q S, the block substitution for E, tril(Q K^T) E, K^T E.
//  * prep waves (NS, NS+1): one chunk ahead of the scan they move the chunk's
//    Q, K, V tile and beta from registers (prefetched a chunk ahead) into
//    LDS, form the Gram tiles (wave NS) and the Q K^T tiles (wave NS+1),
//    lambda, alpha and T_ii; they also write the previous chunk's output from
//    an LDS staging tile to HBM with full-width stores.
// The two groups meet at one workgroup barrier per chunk; the two prep waves
// order their own LDS hand-offs with a counter in LDS.  Every MFMA operand is
// read from LDS ahead of the MFMAs that use it, so the matrix pipe is not
// left waiting on one LDS round trip per instruction.
#include "efla_device.h"
#include "efla_launch.h"

namespace efla {

namespace {

using bf = __bf16;

constexpr int NP = 2;                 // prep waves per workgroup
constexpr int kSpinMax = 1 << 22;     // bound on the prep-wave wait (never reached in practice)

template <int DK, int DV, int C, int NS>
struct FusedLayout {
    static constexpr int TV = 16 * NS;
    static constexpr int MC = C / 16;
    static constexpr int NW = NS + NP;
    static constexpr int LDK = DK + 8, LDV = TV + 8, LDC = C + 8, LDT = 16 + 8, LDD = 20;
    // one chunk of inputs
    static constexpr size_t bQ = 0;
    static constexpr size_t bK = bQ + 2 * C * LDK;
    static constexpr size_t bV = bK + 2 * C * LDK;
    static constexpr size_t bBeta = bV + 2 * C * LDV;
    static constexpr size_t inBytes = (bBeta + 4 * C + 15) / 16 * 16;
    // one chunk of chunk-local quantities
    static constexpr size_t pGb = 0;                          // bf16 G, blocks below the diagonal
    static constexpr size_t pA = pGb + 2 * C * LDC;           // bf16 tril(Q K^T)
    static constexpr size_t pTd = pA + 2 * C * LDC;           // bf16 T_ii: row i -> T_{i/16}[i%16][:]
    static constexpr size_t pGt = pTd + 2 * C * LDT;          // fp32 G_bb transposed: [b][col][row]
    static constexpr size_t pLam = pGt + 4 * MC * 16 * LDD;   // fp32 lambda
    static constexpr size_t pAl = pLam + 4 * C;               // fp32 alpha
    static constexpr size_t prepBytes = (pAl + 4 * C + 15) / 16 * 16;
    // output staging tile
    static constexpr size_t oBytes = (2 * C * LDV + 15) / 16 * 16;
    static constexpr size_t offIn = 0;
    static constexpr size_t offPrep = 2 * inBytes;
    static constexpr size_t offO = offPrep + 2 * prepBytes;
    static constexpr size_t offCtr = offO + 2 * oBytes;
    static constexpr size_t bytes = offCtr + 16;
};

__device__ __forceinline__ bf16x4 zb4() { return to_bf16x4(zero4()); }

// a if c, else zeros (component-wise, so it stays in registers)
__device__ __forceinline__ uint4 keep(bool c, uint4 a)
{
    return make_uint4(c ? a.x : 0u, c ? a.y : 0u, c ? a.z : 0u, c ? a.w : 0u);
}

// MFMA operand for row tile `mt` and 32-wide k-block `s` of an LDS matrix
// (element (i,k) at M[i*ld+k], or M[k*ld+i] when STRIDED), k in the PERM
// order of an acc tile: {32s+4g..+3, 32s+16+4g..+3}.  KT = 16-wide k tiles.
template <bool STRIDED, int KT>
__device__ __forceinline__ bf16x8 a_perm(const bf *M, int ld, int mt, int s)
{
    const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    const int i = 16 * mt + l16;
    const bf16x4 a1 = run4<STRIDED>(M, ld, i, 32 * s + 4 * g);
    const bf16x4 a2 = (2 * s + 1 < KT) ? run4<STRIDED>(M, ld, i, 32 * s + 16 + 4 * g) : zb4();
    return cat(a1, a2);
}

// Same, NAT order {32s+8g..+7}: both operands of a product read from LDS.
template <int K>
__device__ __forceinline__ bf16x8 a_nat(const bf *M, int ld, int row, int s)
{
    const int g = (threadIdx.x & 63) >> 4;
    const int k = 32 * s + 8 * g;
    if (k >= K) return cat(zb4(), zb4());
    return cat(run4<false>(M, ld, row, k), run4<false>(M, ld, row, k + 4));
}

// B operand (PERM order) from KT acc tiles: k-block s = tiles 2s, 2s+1.
template <int KT>
__device__ __forceinline__ bf16x8 b_acc(const f32x4 (&T)[KT], int s)
{
    return cat(to_bf16x4(T[2 * s]), (2 * s + 1 < KT) ? to_bf16x4(T[2 * s + 1]) : zb4());
}

// One chunk's Q, K, V tile and beta in registers of the prep waves.
template <int DK, int DV, int C, int NS>
struct ChunkRegs {
    using Lay = FusedLayout<DK, DV, C, NS>;
    static constexpr int PT = 64 * NP, TV = Lay::TV;
    static constexpr int VQ = C * DK / 8, VV = C * TV / 8;
    static constexpr int PQ = (VQ + PT - 1) / PT, PV = (VV + PT - 1) / PT;
    uint4 q[PQ], k[PQ], v[PV];
    float beta;

    // pt: thread index inside the prep group (0 .. 127).  Branch-free: rows
    // past `valid` (>= 1) re-read row valid-1 and are zeroed afterwards, so
    // every lane issues the same loads and the compiler can count them when
    // it places the waits for this chunk behind later loads and stores.
    __device__ __forceinline__ void load(int pt, const bf *gq, const bf *gk, const bf *gv,
                                         const float *gb, int valid)
    {
#pragma unroll
        for (int i = 0; i < PQ; ++i) {
            const int idx = min(pt + i * PT, VQ - 1), row = idx / (DK / 8), cv = idx % (DK / 8);
            const int rc = min(row, valid - 1);
            const uint4 a = *reinterpret_cast<const uint4 *>(gq + (long)rc * DK + cv * 8);
            const uint4 b = *reinterpret_cast<const uint4 *>(gk + (long)rc * DK + cv * 8);
            q[i] = keep(row < valid, a);
            k[i] = keep(row < valid, b);
        }
#pragma unroll
        for (int i = 0; i < PV; ++i) {
            const int idx = min(pt + i * PT, VV - 1), row = idx / (TV / 8), cv = idx % (TV / 8);
            const int rc = min(row, valid - 1);
            const uint4 a = *reinterpret_cast<const uint4 *>(gv + (long)rc * DV + cv * 8);
            v[i] = keep(row < valid, a);
        }
        const float bt = gb[min(pt, valid - 1)];
        beta = pt < valid ? bt : 0.f;
    }

    __device__ __forceinline__ void store(int pt, char *buf) const
    {
        bf *sQ = reinterpret_cast<bf *>(buf + Lay::bQ);
        bf *sK = reinterpret_cast<bf *>(buf + Lay::bK);
        bf *sV = reinterpret_cast<bf *>(buf + Lay::bV);
        float *sB = reinterpret_cast<float *>(buf + Lay::bBeta);
#pragma unroll
        for (int i = 0; i < PQ; ++i) {
            const int idx = pt + i * PT, row = idx / (DK / 8), cv = idx % (DK / 8);
            if (VQ % PT == 0 || idx < VQ) {
                *reinterpret_cast<uint4 *>(sQ + row * Lay::LDK + cv * 8) = q[i];
                *reinterpret_cast<uint4 *>(sK + row * Lay::LDK + cv * 8) = k[i];
            }
        }
#pragma unroll
        for (int i = 0; i < PV; ++i) {
            const int idx = pt + i * PT, row = idx / (TV / 8), cv = idx % (TV / 8);
            if (VV % PT == 0 || idx < VV) *reinterpret_cast<uint4 *>(sV + row * Lay::LDV + cv * 8) = v[i];
        }
        if (pt < C) sB[pt] = beta;
    }
};

// Ordering point between the prep waves only: every prep wave's LDS writes
// issued before the call are visible to the other prep wave after it.
__device__ __forceinline__ void prep_sync(unsigned *ctr, unsigned &target)
{
    target += NP;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    for (int it = 0; it < kSpinMax; ++it) {
        if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// Prep step 1.  Prep wave 0: Gram tiles G = K K^T below and on the diagonal
// (diagonal blocks transposed in fp32 with lambda from their diagonal, the
// others in bf16).  Prep wave 1: tril(Q K^T) (diagonal tiles masked).
template <int DK, int DV, int C, int NS>
__device__ __forceinline__ void prep_tiles(int p, const char *in, char *prep)
{
    using Lay = FusedLayout<DK, DV, C, NS>;
    constexpr int MC = Lay::MC, NKS = (DK + 31) / 32;
    const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    const bf *sQ = reinterpret_cast<const bf *>(in + Lay::bQ);
    const bf *sK = reinterpret_cast<const bf *>(in + Lay::bK);
    bf16x8 kb[MC][NKS];   // K row blocks as operands (NAT order)
#pragma unroll
    for (int b = 0; b < MC; ++b)
#pragma unroll
        for (int s = 0; s < NKS; ++s) kb[b][s] = a_nat<DK>(sK, Lay::LDK, 16 * b + l16, s);
    if (p == 0) {
        bf *sGb = reinterpret_cast<bf *>(prep + Lay::pGb);
        float *sGt = reinterpret_cast<float *>(prep + Lay::pGt);
        float *sLam = reinterpret_cast<float *>(prep + Lay::pLam);
#pragma unroll
        for (int it = 0; it < MC; ++it)
#pragma unroll
            for (int jt = 0; jt <= it; ++jt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s < NKS; ++s) acc = mma(kb[it][s], kb[jt][s], acc);
                if (it == jt) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 4 * g + r;
                        sGt[(it * 16 + l16) * Lay::LDD + row] = acc[r];
                        if (row == l16) sLam[16 * it + row] = acc[r];
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sGb[(16 * it + 4 * g + r) * Lay::LDC + 16 * jt + l16] = static_cast<bf>(acc[r]);
                }
            }
    } else {
        bf *sA = reinterpret_cast<bf *>(prep + Lay::pA);
#pragma unroll
        for (int it = 0; it < MC; ++it) {
            bf16x8 qa[NKS];
#pragma unroll
            for (int s = 0; s < NKS; ++s) qa[s] = a_nat<DK>(sQ, Lay::LDK, 16 * it + l16, s);
#pragma unroll
            for (int jt = 0; jt <= it; ++jt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s < NKS; ++s) acc = mma(qa[s], kb[jt][s], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * it + 4 * g + r, col = 16 * jt + l16;
                    sA[row * Lay::LDC + col] = static_cast<bf>(col <= row ? acc[r] : 0.f);
                }
            }
        }
    }
}

// Prep step 2: alpha, then T_ii of the blocks this prep wave owns (block b on
// prep wave b % NP, lane group (b / NP) % 4; lane l16 owns column l16).
// Right-looking substitution: once T[i][j] is known it is eliminated from
// every later row, so each of the 16 steps carries independent FMAs.
template <int DK, int DV, int C, int NS>
__device__ __forceinline__ void prep_diag(int p, const char *in, char *prep)
{
    using Lay = FusedLayout<DK, DV, C, NS>;
    constexpr int MC = Lay::MC;
    const int lane = threadIdx.x & 63;
    const float *sB = reinterpret_cast<const float *>(in + Lay::bBeta);
    const float *sGt = reinterpret_cast<const float *>(prep + Lay::pGt);
    const float *sLam = reinterpret_cast<const float *>(prep + Lay::pLam);
    float *sAl = reinterpret_cast<float *>(prep + Lay::pAl);
    bf *sTd = reinterpret_cast<bf *>(prep + Lay::pTd);
    // alpha of the tokens in this wave's blocks (lane = token)
    if (lane < C && ((lane >> 4) % NP) == p) sAl[lane] = efla_alpha(sB[lane], sLam[lane]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int b = p + NP * (lane >> 4);
    if (b < MC) {
        const int j = lane & 15;
        const float *Gt = sGt + b * 16 * Lay::LDD;
        float al[16];
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
            const float4 x = *reinterpret_cast<const float4 *>(sAl + 16 * b + i);
            al[i] = x.x; al[i + 1] = x.y; al[i + 2] = x.z; al[i + 3] = x.w;
        }
        float acc[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) acc[m] = (m == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float gc[16];   // column i of G_bb: gc[m] = G[16b+m][16b+i]
#pragma unroll
            for (int m = 0; m < 16; m += 4) {
                const float4 x = *reinterpret_cast<const float4 *>(Gt + i * Lay::LDD + m);
                gc[m] = x.x; gc[m + 1] = x.y; gc[m + 2] = x.z; gc[m + 3] = x.w;
            }
            const float t = al[i] * acc[i];
            sTd[(16 * b + i) * Lay::LDT + j] = static_cast<bf>(t);
#pragma unroll
            for (int m = i + 1; m < 16; ++m) acc[m] = fmaf(-gc[m], t, acc[m]);
        }
    }
}

// State of a prep wave: buffers, sequence pointers and its prep_sync target.
template <int DK, int DV, int C, int NS>
struct PrepCtx {
    using Lay = FusedLayout<DK, DV, C, NS>;
    char *smem;
    const bf *qb, *kb, *vb;
    const float *bb;
    bf *ob;
    int L, nchunks, p, pt;
    unsigned target;
    __device__ __forceinline__ char *inb(int i) const { return smem + Lay::offIn + i * Lay::inBytes; }
    __device__ __forceinline__ char *prb(int i) const { return smem + Lay::offPrep + i * Lay::prepBytes; }
    __device__ __forceinline__ bf *obuf(int i) const
    {
        return reinterpret_cast<bf *>(smem + Lay::offO + i * Lay::oBytes);
    }
    __device__ __forceinline__ unsigned *ctr() const
    {
        return reinterpret_cast<unsigned *>(smem + Lay::offCtr);
    }
    __device__ __forceinline__ int valid_of(int c) const { return min(C, L - c * C); }
};

// Chunks past the end re-load the last chunk (never stored), keeping the
// number of loads in flight the same on every path.
template <int DK, int DV, int C, int NS>
__device__ __attribute__((always_inline)) inline void prep_load(const PrepCtx<DK, DV, C, NS> &x,
                                                                ChunkRegs<DK, DV, C, NS> &r, int n)
{
    n = min(n, x.nchunks - 1);
    const long off = (long)n * C;
    r.load(x.pt, x.qb + off * DK, x.kb + off * DK, x.vb + off * DV, x.bb + off, x.valid_of(n));
}

// A chunk's output rows, staged in LDS by the scan waves, to HBM; rows past
// `valid` rewrite row valid-1 with its own value.
template <int DK, int DV, int C, int NS>
__device__ __attribute__((always_inline)) inline void prep_store_out(const PrepCtx<DK, DV, C, NS> &x,
                                                                     int n)
{
    using Lay = FusedLayout<DK, DV, C, NS>;
    constexpr int VPR = Lay::TV / 8, NV = C * VPR, PT = 64 * NP;
    const bf *os = x.obuf(n & 1);
    const int valid = x.valid_of(n);
    bf *dst = x.ob + (long)n * C * DV;
#pragma unroll
    for (int i = 0; i < (NV + PT - 1) / PT; ++i) {
        const int idx = min(x.pt + i * PT, NV - 1);
        const int row = min(idx / VPR, valid - 1), cv = idx % VPR;
        *reinterpret_cast<uint4 *>(dst + (long)row * DV + cv * 8) =
            *reinterpret_cast<const uint4 *>(os + row * Lay::LDV + cv * 8);
    }
}

// Prepare chunk n from input buffer n & 1.
template <int DK, int DV, int C, int NS>
__device__ __attribute__((always_inline)) inline void prep_chunk(PrepCtx<DK, DV, C, NS> &x, int n)
{
    prep_sync(x.ctr(), x.target);
    prep_tiles<DK, DV, C, NS>(x.p, x.inb(n & 1), x.prb(n & 1));
    prep_sync(x.ctr(), x.target);
    prep_diag<DK, DV, C, NS>(x.p, x.inb(n & 1), x.prb(n & 1));
}

// One chunk of the scan for the calling wave (16 state columns).
template <int DK, int DV, int C, int NS>
__device__ __attribute__((always_inline)) inline void scan_chunk(f32x4 (&S)[DK / 16], const char *in,
                                                                 const char *pr, bf *os, int wv)
{
    using Lay = FusedLayout<DK, DV, C, NS>;
    constexpr int MC = Lay::MC, MK = DK / 16, NKS = (MK + 1) / 2, NKC = (MC + 1) / 2;
    const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    const bf *sQ = reinterpret_cast<const bf *>(in + Lay::bQ);
    const bf *sK = reinterpret_cast<const bf *>(in + Lay::bK);
    const bf *sV = reinterpret_cast<const bf *>(in + Lay::bV);
    const bf *sGb = reinterpret_cast<const bf *>(pr + Lay::pGb);
    const bf *sA = reinterpret_cast<const bf *>(pr + Lay::pA);
    const bf *sTd = reinterpret_cast<const bf *>(pr + Lay::pTd);

    // V in acc layout
    float vv[MC][4];
#pragma unroll
    for (int mt = 0; mt < MC; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) vv[mt][r] = to_f32(sV[(16 * mt + 4 * g + r) * Lay::LDV + 16 * wv + l16]);

    // X = K S and O = Q S, k-block by k-block with the next block's operands
    // already in flight
    bf16x8 bS[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) bS[s] = b_acc(S, s);
    f32x4 X[MC], O[MC];
#pragma unroll
    for (int mt = 0; mt < MC; ++mt) X[mt] = O[mt] = zero4();
    bf16x8 ak[2][MC], aq[2][MC];
#pragma unroll
    for (int mt = 0; mt < MC; ++mt) {
        ak[0][mt] = a_perm<false, MK>(sK, Lay::LDK, mt, 0);
        aq[0][mt] = a_perm<false, MK>(sQ, Lay::LDK, mt, 0);
    }
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        if (s + 1 < NKS) {
#pragma unroll
            for (int mt = 0; mt < MC; ++mt) {
                ak[(s + 1) & 1][mt] = a_perm<false, MK>(sK, Lay::LDK, mt, s + 1);
                aq[(s + 1) & 1][mt] = a_perm<false, MK>(sQ, Lay::LDK, mt, s + 1);
            }
        }
#pragma unroll
        for (int mt = 0; mt < MC; ++mt) {
            X[mt] = mma(ak[s & 1][mt], bS[s], X[mt]);
            O[mt] = mma(aq[s & 1][mt], bS[s], O[mt]);
        }
    }

    // operands of the rest of the chunk, loaded before the dependent chain
    bf16x8 ga[MC * NKC];                  // G_{i, 2s..2s+1} for i >= 1
#pragma unroll
    for (int i = 1; i < MC; ++i)
#pragma unroll
        for (int s = 0; 2 * s < i; ++s) {
            const bool two = 2 * s + 1 < i;
            const bf *arow = sGb + (16 * i + l16) * Lay::LDC + 32 * s + 4 * g;
            ga[i * NKC + s] = cat(*reinterpret_cast<const bf16x4 *>(arow),
                                  two ? *reinterpret_cast<const bf16x4 *>(arow + 16) : zb4());
        }
    bf16x4 ta[MC];
#pragma unroll
    for (int i = 0; i < MC; ++i) ta[i] = *reinterpret_cast<const bf16x4 *>(sTd + (16 * i + l16) * Lay::LDT + 4 * g);
    bf16x8 aa[MC * NKC];                  // tril(Q K^T), block lower triangle
#pragma unroll
    for (int mt = 0; mt < MC; ++mt)
#pragma unroll
        for (int s = 0; 2 * s <= mt; ++s) aa[mt * NKC + s] = a_perm<false, MC>(sA, Lay::LDC, mt, s);
    bf16x8 akt[MK * NKC];                 // K^T
#pragma unroll
    for (int mt = 0; mt < MK; ++mt)
#pragma unroll
        for (int s = 0; s < NKC; ++s) akt[mt * NKC + s] = a_perm<true, MC>(sK, Lay::LDK, mt, s);

    // E by block substitution
#pragma unroll
    for (int mt = 0; mt < MC; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) X[mt][r] = vv[mt][r] - X[mt][r];
    f32x4 E[MC];
#pragma unroll
    for (int i = 0; i < MC; ++i) {
        f32x4 y = X[i];
#pragma unroll
        for (int s = 0; 2 * s < i; ++s) {   // only blocks m < i of E exist yet
            const bf16x8 be = cat(to_bf16x4(E[2 * s]), 2 * s + 1 < i ? to_bf16x4(E[2 * s + 1]) : zb4());
            y -= mma(ga[i * NKC + s], be, zero4());
        }
        E[i] = mma(cat(ta[i], zb4()), cat(to_bf16x4(y), zb4()), zero4());
    }

    // O += tril(Q K^T) E;  S += K^T E
    bf16x8 bE[NKC];
#pragma unroll
    for (int s = 0; s < NKC; ++s) bE[s] = b_acc(E, s);
#pragma unroll
    for (int s = 0; s < NKC; ++s)
#pragma unroll
        for (int mt = 0; mt < MC; ++mt)
            if (2 * s <= mt) O[mt] = mma(aa[mt * NKC + s], bE[s], O[mt]);
#pragma unroll
    for (int s = 0; s < NKC; ++s)
#pragma unroll
        for (int mt = 0; mt < MK; ++mt) S[mt] = mma(akt[mt * NKC + s], bE[s], S[mt]);

#pragma unroll
    for (int mt = 0; mt < MC; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            os[(16 * mt + 4 * g + r) * Lay::LDV + 16 * wv + l16] = static_cast<bf>(O[mt][r]);
}

template <int DK, int DV, int C, int NS>
__global__ __launch_bounds__(64 * (NS + NP)) void fused_kernel(
    const bf *__restrict__ q, const bf *__restrict__ k, const bf *__restrict__ v,
    const float *__restrict__ beta, const float *__restrict__ S0, bf *__restrict__ o,
    float *__restrict__ SL, int L, int nchunks)
{
    using Lay = FusedLayout<DK, DV, C, NS>;
    constexpr int TV = Lay::TV, NTILE = DV / TV, MK = DK / 16;
    extern __shared__ __align__(16) char smem[];

    int bh, tile;
    xcd_map(blockIdx.x, gridDim.x, NTILE, bh, tile);
    const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long tokb = (long)bh * L;

    if (threadIdx.x == 0) *reinterpret_cast<unsigned *>(smem + Lay::offCtr) = 0u;
    // upper tiles of tril(Q K^T) stay zero for the whole kernel
    for (int b = 0; b < 2; ++b) {
        bf *sA = reinterpret_cast<bf *>(smem + Lay::offPrep + b * Lay::prepBytes + Lay::pA);
        for (int i = threadIdx.x; i < C * C; i += 64 * Lay::NW) {
            const int r = i / C, cc = i - r * C;
            if ((cc >> 4) > (r >> 4)) sA[r * Lay::LDC + cc] = static_cast<bf>(0.f);
        }
    }
    __syncthreads();

    if (wv < NS) {
        // ------------------------------------------------------------ scan waves
        const int col = tile * TV + 16 * wv + l16;
        f32x4 S[MK];
        const long sbase = (long)bh * DK * DV;
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[mk][r] = S0 ? S0[sbase + (16 * mk + 4 * g + r) * DV + col] : 0.f;
        __syncthreads();   // prologue: chunk 0 prepared
        for (int c = 0; c < nchunks; ++c) {
            scan_chunk<DK, DV, C, NS>(S, smem + Lay::offIn + (c & 1) * Lay::inBytes,
                                      smem + Lay::offPrep + (c & 1) * Lay::prepBytes,
                                      reinterpret_cast<bf *>(smem + Lay::offO + (c & 1) * Lay::oBytes),
                                      wv);
            __syncthreads();
        }
        __syncthreads();   // epilogue: the prep waves write the last chunk's output
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int r = 0; r < 4; ++r) SL[sbase + (16 * mk + 4 * g + r) * DV + col] = S[mk][r];
    } else {
        // ------------------------------------------------------------ prep waves
        PrepCtx<DK, DV, C, NS> x{smem, q + tokb * DK, k + tokb * DK, v + tokb * DV + tile * TV,
                                 beta + tokb, o + tokb * DV + tile * TV, L, nchunks, wv - NS,
                                 (int)threadIdx.x - 64 * NS, 0u};
        ChunkRegs<DK, DV, C, NS> r;   // holds chunk c+1 at the start of interval c
        prep_load(x, r, 0);
        r.store(x.pt, x.inb(0));
        prep_load(x, r, 1);
        prep_chunk(x, 0);
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            if (c + 1 < nchunks) {
                r.store(x.pt, x.inb((c + 1) & 1));
                prep_load(x, r, c + 2);
                prep_chunk(x, c + 1);
            }
            if (c > 0) prep_store_out(x, c - 1);
            __syncthreads();
        }
        __syncthreads();
        prep_store_out(x, nchunks - 1);
    }
}

template <int DK, int DV, int C, int NS>
hipError_t launch_fused(const void *q, const void *k, const void *v, const float *beta,
                        const float *S0, void *o, float *SL, int BH, int L, hipStream_t st)
{
    using Lay = FusedLayout<DK, DV, C, NS>;
    static_assert(Lay::bytes <= 160 * 1024, "fused kernel LDS budget");
    constexpr int NTILE = DV / Lay::TV;
    const int nchunks = (L + C - 1) / C;
    if (BH == 0 || nchunks == 0) return hipSuccess;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&fused_kernel<DK, DV, C, NS>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((fused_kernel<DK, DV, C, NS>), dim3((unsigned)(BH * NTILE)),
                       dim3(64 * Lay::NW), Lay::bytes, st, static_cast<const bf *>(q),
                       static_cast<const bf *>(k), static_cast<const bf *>(v), beta, S0,
                       static_cast<bf *>(o), SL, L, nchunks);
    return hipGetLastError();
}

template <int DK, int DV, int C>
hipError_t launch_fused_ns(const void *q, const void *k, const void *v, const float *beta,
                           const float *S0, void *o, float *SL, int BH, int L, int ns,
                           hipStream_t st)
{
    if (ns <= 0) ns = DV >= 32 ? 2 : 1;
    if (ns >= 2 && DV >= 32) return launch_fused<DK, DV, C, 2>(q, k, v, beta, S0, o, SL, BH, L, st);
    return launch_fused<DK, DV, C, 1>(q, k, v, beta, S0, o, SL, BH, L, st);
}

}  // namespace

bool fused_supported(bool bf16, int dk, int dv, int chunk)
{
    (void)dk;
    (void)dv;
    (void)chunk;
    return bf16;
}

hipError_t dispatch_fused(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                          const void *v, const float *beta, const float *S0, void *o, float *SL,
                          int BH, int L, int ns, hipStream_t st)
{
    if (!bf16) return hipErrorInvalidValue;
#define CASE(DKV, DVV, CC)                                                                      \
    if (dk == DKV && dv == DVV && chunk == CC)                                                  \
        return launch_fused_ns<DKV, DVV, CC>(q, k, v, beta, S0, o, SL, BH, L, ns, st);
    EFLA_SHAPE_CASES(CASE)
#undef CASE
    return hipErrorInvalidValue;
}

}  // namespace efla
