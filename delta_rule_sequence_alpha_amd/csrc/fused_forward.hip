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
//  * prep wave NS ("K wave"), one chunk ahead of the scan: moves the chunk's
//    K and beta from registers (prefetched a chunk ahead) into LDS, then forms
//    the Gram tiles, lambda, alpha and every T_ii (one 16-lane group per
//    diagonal block).
//  * prep wave NS+1 ("Q wave"), one chunk ahead: moves Q and the V tile into
//    LDS, writes the previous chunk's output from an LDS staging tile to HBM
//    with full-width stores, then forms tril(Q K^T) once the K wave has
//    signalled that K is in LDS.
// The scan and prep groups meet at one workgroup barrier per chunk; the only
// other hand-off is the K wave's one-way signal to the Q wave, a counter in
// LDS.  The scan reads K^T operands with the transposing LDS read of gfx950.
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

// Which d_k row each accumulator row of the state holds.  S is kept as
// DK/16 accumulator tiles; tile t = 2s + h (h = 0, 1) and acc row i = 4q + e
// hold d_k row 32s + 8q + 4h + e.  Then the eight values lane group g feeds
// an MFMA for k-block s -- rows 4g..4g+3 of tiles 2s and 2s+1 -- are the
// eight consecutive d_k rows 32s + 8g .. 32s + 8g + 7, so the matching A
// operand (K or Q) is one contiguous 16-byte LDS read.  d_k = 16: identity.
template <int DK>
__device__ __forceinline__ int srow(int t, int i)
{
    if constexpr (DK < 32) return i;
    return 32 * (t >> 1) + 8 * (i >> 2) + 4 * (t & 1) + (i & 3);
}

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

// Row tile `mt`, k-block `s` of Q or K as the A operand against the state
// (rows in the srow order): one 16-byte read of d_k columns 32s+8g..+7.
template <int DK>
__device__ __forceinline__ bf16x8 a_row(const bf *M, int ld, int mt, int s)
{
    if constexpr (DK < 32) return a_perm<false, DK / 16>(M, ld, mt, s);
    const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    return *reinterpret_cast<const bf16x8 *>(M + (16 * mt + l16) * ld + 32 * s + 8 * g);
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

// One chunk's inputs in the registers of one prep wave: the K wave holds K
// and beta, the Q wave Q and the V tile.  Row-major 16-byte vectors, lane t
// taking vectors t, t+64, ...
template <int DK, int DV, int C, int NS>
struct ChunkRegs {
    using Lay = FusedLayout<DK, DV, C, NS>;
    static constexpr int TV = Lay::TV;
    static constexpr int VM = C * DK / 8, VV = C * TV / 8;       // vectors of K (or Q), of V
    static constexpr int PM = (VM + 63) / 64, PV = (VV + 63) / 64;
    uint4 m[PM], v[PV];
    float beta;

    // Branch-free: rows past `valid` (>= 1) re-read row valid-1 and are
    // zeroed afterwards, so every lane issues the same loads and the compiler
    // can count them when it places waits behind later loads and stores.
    __device__ __forceinline__ void load(bool kwave, int lane, const bf *gq, const bf *gk,
                                         const bf *gv, const float *gb, int valid)
    {
        const bf *gm = kwave ? gk : gq;
        if (valid >= C) {   // full chunk: plain row-major loads, same count as below
#pragma unroll
            for (int i = 0; i < PM; ++i) {
                const int idx = min(lane + i * 64, VM - 1);
                m[i] = *reinterpret_cast<const uint4 *>(gm + idx * 8);
            }
            if (kwave) {
                beta = gb[min(lane, C - 1)];
            } else {
#pragma unroll
                for (int i = 0; i < PV; ++i) {
                    const int idx = min(lane + i * 64, VV - 1), row = idx / (TV / 8), cv = idx % (TV / 8);
                    v[i] = *reinterpret_cast<const uint4 *>(gv + (long)row * DV + cv * 8);
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < PM; ++i) {
            const int idx = min(lane + i * 64, VM - 1), row = idx / (DK / 8), cv = idx % (DK / 8);
            const uint4 a = *reinterpret_cast<const uint4 *>(gm + (long)min(row, valid - 1) * DK + cv * 8);
            m[i] = keep(row < valid, a);
        }
        if (kwave) {
            const float bt = gb[min(lane, valid - 1)];
            beta = lane < valid ? bt : 0.f;
        } else {
#pragma unroll
            for (int i = 0; i < PV; ++i) {
                const int idx = min(lane + i * 64, VV - 1), row = idx / (TV / 8), cv = idx % (TV / 8);
                const uint4 a = *reinterpret_cast<const uint4 *>(gv + (long)min(row, valid - 1) * DV + cv * 8);
                v[i] = keep(row < valid, a);
            }
        }
    }

    __device__ __forceinline__ void store(bool kwave, int lane, char *buf) const
    {
        bf *sM = reinterpret_cast<bf *>(buf + (kwave ? Lay::bK : Lay::bQ));
#pragma unroll
        for (int i = 0; i < PM; ++i) {
            const int idx = lane + i * 64, row = idx / (DK / 8), cv = idx % (DK / 8);
            if (VM % 64 == 0 || idx < VM) *reinterpret_cast<uint4 *>(sM + row * Lay::LDK + cv * 8) = m[i];
        }
        if (kwave) {
            if (lane < C) reinterpret_cast<float *>(buf + Lay::bBeta)[lane] = beta;
        } else {
            bf *sV = reinterpret_cast<bf *>(buf + Lay::bV);
#pragma unroll
            for (int i = 0; i < PV; ++i) {
                const int idx = lane + i * 64, row = idx / (TV / 8), cv = idx % (TV / 8);
                if (VV % 64 == 0 || idx < VV) *reinterpret_cast<uint4 *>(sV + row * Lay::LDV + cv * 8) = v[i];
            }
        }
    }
};

// One-way hand-off from the K wave to the Q wave: the K wave's LDS writes
// issued before k_signal() are visible to the Q wave after its matching
// q_wait().  The wait is bounded; the counter only grows.
__device__ __forceinline__ void k_signal(unsigned *ctr)
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void q_wait(unsigned *ctr, unsigned target)
{
    for (int it = 0; it < kSpinMax; ++it) {
        if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// K wave, step 1: Gram tiles G = K K^T on and below the diagonal (diagonal
// blocks transposed in fp32 with lambda from their diagonal, the others in
// bf16).  All operands are read first, then the MFMAs of every tile run
// k-block by k-block, so no tile waits on another's accumulation chain.
template <int DK, int DV, int C, int NS>
__device__ __forceinline__ void prep_gram(const char *in, char *prep)
{
    using Lay = FusedLayout<DK, DV, C, NS>;
    constexpr int MC = Lay::MC, NKS = (DK + 31) / 32, NT = MC * (MC + 1) / 2;
    const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    const bf *sK = reinterpret_cast<const bf *>(in + Lay::bK);
    bf *sGb = reinterpret_cast<bf *>(prep + Lay::pGb);
    float *sGt = reinterpret_cast<float *>(prep + Lay::pGt);
    float *sLam = reinterpret_cast<float *>(prep + Lay::pLam);
    bf16x8 kb[MC][NKS];   // K row blocks as operands (NAT order)
#pragma unroll
    for (int b = 0; b < MC; ++b)
#pragma unroll
        for (int s = 0; s < NKS; ++s) kb[b][s] = a_nat<DK>(sK, Lay::LDK, 16 * b + l16, s);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = zero4();
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        int t = 0;
#pragma unroll
        for (int it = 0; it < MC; ++it)
#pragma unroll
            for (int jt = 0; jt <= it; ++jt, ++t) acc[t] = mma(kb[it][s], kb[jt][s], acc[t]);
    }
    __builtin_amdgcn_sched_barrier(0);
    int t = 0;
#pragma unroll
    for (int it = 0; it < MC; ++it)
#pragma unroll
        for (int jt = 0; jt <= it; ++jt, ++t) {
            if (it == jt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * g + r;
                    sGt[(it * 16 + l16) * Lay::LDD + row] = acc[t][r];
                    if (row == l16) sLam[16 * it + row] = acc[t][r];
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sGb[(16 * it + 4 * g + r) * Lay::LDC + 16 * jt + l16] = static_cast<bf>(acc[t][r]);
            }
        }
}

// Q wave: tril(Q K^T), diagonal tiles masked; operands first, as above.
template <int DK, int DV, int C, int NS>
__device__ __forceinline__ void prep_qk(const char *in, char *prep)
{
    using Lay = FusedLayout<DK, DV, C, NS>;
    constexpr int MC = Lay::MC, NKS = (DK + 31) / 32, NT = MC * (MC + 1) / 2;
    const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    const bf *sQ = reinterpret_cast<const bf *>(in + Lay::bQ);
    const bf *sK = reinterpret_cast<const bf *>(in + Lay::bK);
    bf *sA = reinterpret_cast<bf *>(prep + Lay::pA);
    bf16x8 kb[MC][NKS], qa[MC][NKS];
#pragma unroll
    for (int b = 0; b < MC; ++b)
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            kb[b][s] = a_nat<DK>(sK, Lay::LDK, 16 * b + l16, s);
            qa[b][s] = a_nat<DK>(sQ, Lay::LDK, 16 * b + l16, s);
        }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = zero4();
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        int t = 0;
#pragma unroll
        for (int it = 0; it < MC; ++it)
#pragma unroll
            for (int jt = 0; jt <= it; ++jt, ++t) acc[t] = mma(qa[it][s], kb[jt][s], acc[t]);
    }
    __builtin_amdgcn_sched_barrier(0);
    int t = 0;
#pragma unroll
    for (int it = 0; it < MC; ++it)
#pragma unroll
        for (int jt = 0; jt <= it; ++jt, ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * it + 4 * g + r, col = 16 * jt + l16;
                sA[row * Lay::LDC + col] = static_cast<bf>(col <= row ? acc[t][r] : 0.f);
            }
}

// K wave, step 2: alpha (lane = token), then every T_ii, lane group b owning
// block b and lane l16 its column l16.  Right-looking substitution: once
// T[i][j] is known it is eliminated from every later row, so each of the 16
// steps carries independent FMAs; the next step's column of G is read while
// the current one is applied.
template <int DK, int DV, int C, int NS>
__device__ __forceinline__ void prep_diag(const char *in, char *prep)
{
    using Lay = FusedLayout<DK, DV, C, NS>;
    constexpr int MC = Lay::MC;
    const int lane = threadIdx.x & 63;
    const float *sB = reinterpret_cast<const float *>(in + Lay::bBeta);
    const float *sGt = reinterpret_cast<const float *>(prep + Lay::pGt);
    const float *sLam = reinterpret_cast<const float *>(prep + Lay::pLam);
    float *sAl = reinterpret_cast<float *>(prep + Lay::pAl);
    bf *sTd = reinterpret_cast<bf *>(prep + Lay::pTd);
    if (lane < C) sAl[lane] = efla_alpha(sB[lane], sLam[lane]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int b = lane >> 4;
    if (b < MC) {
        const int j = lane & 15;
        const float *Gt = sGt + b * 16 * Lay::LDD;
        float al[16];
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
            const float4 x = *reinterpret_cast<const float4 *>(sAl + 16 * b + i);
            al[i] = x.x; al[i + 1] = x.y; al[i + 2] = x.z; al[i + 3] = x.w;
        }
        // every value the substitution reads, G[m][i] for m > i, loaded up
        // front as float4 groups of column i (rows 4*qq .. 4*qq+3)
        float4 gcol[16][4];
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int qq = (i + 1) / 4; qq < 4; ++qq)
                gcol[i][qq] = *reinterpret_cast<const float4 *>(Gt + i * Lay::LDD + 4 * qq);
        __builtin_amdgcn_sched_barrier(0);
        float acc[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) acc[m] = (m == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float t = al[i] * acc[i];
            sTd[(16 * b + i) * Lay::LDT + j] = static_cast<bf>(t);
#pragma unroll
            for (int m = i + 1; m < 16; ++m) {
                const float4 gv = gcol[i][m >> 2];
                const float gm = (m & 3) == 0 ? gv.x : (m & 3) == 1 ? gv.y : (m & 3) == 2 ? gv.z : gv.w;
                acc[m] = fmaf(-gm, t, acc[m]);
            }
        }
    }
}

// State of a prep wave: buffers, sequence pointers and its role.
template <int DK, int DV, int C, int NS>
struct PrepCtx {
    using Lay = FusedLayout<DK, DV, C, NS>;
    char *smem;
    const bf *qb, *kb, *vb;
    const float *bb;
    bf *ob;
    int L, nchunks, lane;
    bool kwave;
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
    r.load(x.kwave, x.lane, x.qb + off * DK, x.kb + off * DK, x.vb + off * DV, x.bb + off,
           x.valid_of(n));
}

// A chunk's output rows, staged in LDS by the scan waves, to HBM (Q wave);
// rows past `valid` rewrite row valid-1 with its own value.
template <int DK, int DV, int C, int NS>
__device__ __attribute__((always_inline)) inline void prep_store_out(const PrepCtx<DK, DV, C, NS> &x,
                                                                     int n)
{
    using Lay = FusedLayout<DK, DV, C, NS>;
    constexpr int VPR = Lay::TV / 8, NV = C * VPR;
    const bf *os = x.obuf(n & 1);
    const int valid = x.valid_of(n);
    bf *dst = x.ob + (long)n * C * DV;
#pragma unroll
    for (int i = 0; i < (NV + 63) / 64; ++i) {
        const int idx = min(x.lane + i * 64, NV - 1);
        const int row = min(idx / VPR, valid - 1), cv = idx % VPR;
        *reinterpret_cast<uint4 *>(dst + (long)row * DV + cv * 8) =
            *reinterpret_cast<const uint4 *>(os + row * Lay::LDV + cv * 8);
    }
}

// One prep interval for chunk n (its inputs are in r on entry).  Loads of
// chunk n+1 are issued as soon as r has been written to LDS.
template <int DK, int DV, int C, int NS>
__device__ __attribute__((always_inline)) inline void prep_interval(const PrepCtx<DK, DV, C, NS> &x,
                                                                    ChunkRegs<DK, DV, C, NS> &r,
                                                                    int n, int out_chunk)
{
    char *in = x.inb(n & 1);
    char *pr = x.prb(n & 1);
    r.store(x.kwave, x.lane, in);
    prep_load(x, r, n + 1);
    if (x.kwave) {
        k_signal(x.ctr());
        prep_gram<DK, DV, C, NS>(in, pr);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        prep_diag<DK, DV, C, NS>(in, pr);
    } else {
        if (out_chunk >= 0) prep_store_out(x, out_chunk);
        q_wait(x.ctr(), (unsigned)(n + 1));
        prep_qk<DK, DV, C, NS>(in, pr);
    }
}

// transposing LDS read: within each 16-lane group, lane l receives element
// l%4 of the 4 x 16-bit values addressed by lane 4e + l/4, for e = 0..3
__device__ __forceinline__ bf16x4 ds_read_tr(const bf *p)
{
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// K^T operand for state tile mt (d_k rows srow(mt, 0..15)) and token
// k-block s, PERM order: lane (l16, g) gets K[32s+4g+r][srow(mt,l16)] and
// K[32s+16+4g+r][srow(mt,l16)].  srow(mt, 4q..4q+3) are 4 consecutive d_k,
// so lane l16 of the group points the read at K[c0 + l16/4][srow(mt, 4*(l16%4))].
template <int DK, int MC>
__device__ __forceinline__ bf16x8 a_kt(const bf *sK, int ld, int mt, int s)
{
    const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    const bf *base = sK + (32 * s + 4 * g + (l16 >> 2)) * ld + srow<DK>(mt, 4 * (l16 & 3));
    const bf16x4 a1 = ds_read_tr(base);
    const bf16x4 a2 = (2 * s + 1 < MC) ? ds_read_tr(base + 16 * ld) : zb4();
    return cat(a1, a2);
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
        ak[0][mt] = a_row<DK>(sK, Lay::LDK, mt, 0);
        aq[0][mt] = a_row<DK>(sQ, Lay::LDK, mt, 0);
    }
    // reads of k-block s+1 are issued before the MFMAs of block s and kept
    // there, so each MFMA group covers the next group's LDS latency
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        if (s + 1 < NKS) {
#pragma unroll
            for (int mt = 0; mt < MC; ++mt) {
                ak[(s + 1) & 1][mt] = a_row<DK>(sK, Lay::LDK, mt, s + 1);
                aq[(s + 1) & 1][mt] = a_row<DK>(sQ, Lay::LDK, mt, s + 1);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < MC; ++mt) {
            X[mt] = mma(ak[s & 1][mt], bS[s], X[mt]);
            O[mt] = mma(aq[s & 1][mt], bS[s], O[mt]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);

    // E by block substitution on X = V - K S
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
#pragma unroll
    for (int mt = 0; mt < MC; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            X[mt][r] = to_f32(sV[(16 * mt + 4 * g + r) * Lay::LDV + 16 * wv + l16]) - X[mt][r];
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
    __builtin_amdgcn_sched_barrier(0);

    // O += tril(Q K^T) E;  S += K^T E   (operands read a group ahead)
    bf16x8 bE[NKC];
#pragma unroll
    for (int s = 0; s < NKC; ++s) bE[s] = b_acc(E, s);
    bf16x8 aa[MC * NKC];
#pragma unroll
    for (int s = 0; s < NKC; ++s)
#pragma unroll
        for (int mt = 0; mt < MC; ++mt)
            if (2 * s <= mt) aa[mt * NKC + s] = a_perm<false, MC>(sA, Lay::LDC, mt, s);
    constexpr int KG = MK / 2 > 0 ? MK / 2 : 1;   // K^T row tiles per read group
    bf16x8 akt[2][KG];
#pragma unroll
    for (int j = 0; j < KG; ++j) akt[0][j] = a_kt<DK, MC>(sK, Lay::LDK, j, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < NKC; ++s)
#pragma unroll
        for (int mt = 0; mt < MC; ++mt)
            if (2 * s <= mt) O[mt] = mma(aa[mt * NKC + s], bE[s], O[mt]);
    constexpr int NG = (MK + KG - 1) / KG * NKC;   // read groups of K^T
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const int s = gi / ((MK + KG - 1) / KG), mt0 = (gi % ((MK + KG - 1) / KG)) * KG;
        if (gi + 1 < NG) {
            const int s1 = (gi + 1) / ((MK + KG - 1) / KG), mt1 = ((gi + 1) % ((MK + KG - 1) / KG)) * KG;
#pragma unroll
            for (int j = 0; j < KG; ++j)
                if (mt1 + j < MK) akt[(gi + 1) & 1][j] = a_kt<DK, MC>(sK, Lay::LDK, mt1 + j, s1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < KG; ++j)
            if (mt0 + j < MK) S[mt0 + j] = mma(akt[gi & 1][j], bE[s], S[mt0 + j]);
        __builtin_amdgcn_sched_barrier(0);
    }

#pragma unroll
    for (int mt = 0; mt < MC; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            os[(16 * mt + 4 * g + r) * Lay::LDV + 16 * wv + l16] = static_cast<bf>(O[mt][r]);
}

template <int DK, int DV, int C, int NS>
// One workgroup per CU by design (its LDS footprint), one wave per SIMD:
// let the register allocator use the whole register file for latency hiding.
__global__ __launch_bounds__(64 * (NS + NP)) __attribute__((amdgpu_waves_per_eu(1, 1))) void fused_kernel(
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
                S[mk][r] = S0 ? S0[sbase + srow<DK>(mk, 4 * g + r) * DV + col] : 0.f;
        __syncthreads();   // prologue: chunk 0 prepared
        for (int c = 0; c < nchunks; ++c) {
            scan_chunk<DK, DV, C, NS>(S, smem + Lay::offIn + (c & 1) * Lay::inBytes,
                                      smem + Lay::offPrep + (c & 1) * Lay::prepBytes,
                                      reinterpret_cast<bf *>(smem + Lay::offO + (c & 1) * Lay::oBytes),
                                      wv);
            __syncthreads();
        }
        __syncthreads();   // epilogue: the Q wave writes the last chunk's output
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int r = 0; r < 4; ++r) SL[sbase + srow<DK>(mk, 4 * g + r) * DV + col] = S[mk][r];
    } else {
        // ------------------------------------------------------------ prep waves
        const PrepCtx<DK, DV, C, NS> x{smem, q + tokb * DK, k + tokb * DK, v + tokb * DV + tile * TV,
                                       beta + tokb, o + tokb * DV + tile * TV, L, nchunks, lane,
                                       wv == NS};
        ChunkRegs<DK, DV, C, NS> r;   // inputs of the next chunk to prepare
        prep_load(x, r, 0);
        prep_interval(x, r, 0, -1);   // prologue: chunk 0
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            // interval c: the scan works on chunk c; prepare chunk c+1 and write
            // the output of chunk c-1
            if (c + 1 < nchunks) prep_interval(x, r, c + 1, c - 1);
            else if (!x.kwave && c > 0) prep_store_out(x, c - 1);
            __syncthreads();
        }
        __syncthreads();
        if (!x.kwave) prep_store_out(x, nchunks - 1);
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
