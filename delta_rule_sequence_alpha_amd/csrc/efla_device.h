// Device-side building blocks shared by the EFLA kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used throughout (wave64):
//   lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4 (four lane groups).
//   An "acc tile" is the fp32 result of a 16x16 MFMA: lane holds rows 4g+r
//   (r = 0..3) of column l16.
//   v_mfma_f32_16x16x32_bf16: each lane feeds 8 bf16 of A (row l16) and 8 of B
//   (column l16).  v_mfma_f32_16x16x4_f32: one fp32 of each.
//
// The contraction index k may be assigned to (lane group, slot) by any
// bijection, provided A and B use the same one.  Two maps are used:
//   NAT  (natural):  bf16 k = 8g + j                  f32 k = g
//   PERM (acc map):  bf16 k = 16*(j/4) + 4g + (j%4)   f32 k = 4g   (+ r per step)
// PERM is the row order in which an acc tile already sits in the registers,
// so a product whose B operand is an acc tile (the state S, or E) consumes it
// straight from registers without a trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace efla {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <typename T> struct is_bf16_t { static constexpr bool value = false; };
template <> struct is_bf16_t<__bf16> { static constexpr bool value = true; };
template <typename T> constexpr bool is_bf16 = is_bf16_t<T>::value;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return static_cast<T>(x); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x16_bf16: lane feeds 4 bf16 of A (row l16, k = 4g..4g+3)
// and of B (column l16, the same k) -- an acc tile's own layout.
__device__ __forceinline__ f32x4 mma(bf16x4 a, bf16x4 b, f32x4 c)
{
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b)
{
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 v)
{
    return bf16x4{static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]),
                  static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])};
}

// The strided four-element run for a whole 16-lane group in one transposing
// LDS read (ds_read_tr16_b64): with k the same across the group, lane l16
// receives M[(k+e)*ld + i0 + l16] for e = 0..3.  Lane j of the group
// addresses the four consecutive elements at M[(k + j/4)*ld + i0 + 4(j%4)],
// and the read gives lane l16 element l16%4 of the run addressed by lane
// 4e + l16/4.  M must be in LDS; ld and i0 multiples of 4.
__device__ __forceinline__ bf16x4 run4_tr(const __bf16 *M, int ld, int i0, int k)
{
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int l16 = threadIdx.x & 15;
    const __bf16 *p = M + (k + (l16 >> 2)) * ld + i0 + 4 * (l16 & 3);
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// run4 for bf16 operands in LDS, the strided form through run4_tr; idx0 is
// the tile's first row (of A) or column (of B), idx = idx0 + l16.
template <bool STRIDED>
__device__ __forceinline__ bf16x4 run4_lds(const __bf16 *M, int ld, int idx0, int k)
{
    const int l16 = threadIdx.x & 15;
    if constexpr (!STRIDED) return *reinterpret_cast<const bf16x4 *>(M + (idx0 + l16) * ld + k);
    else return run4_tr(M, ld, idx0, k);
}

template <bool STRIDED>
__device__ __forceinline__ float one(const float *M, int ld, int idx, int k)
{
    if constexpr (!STRIDED) return M[idx * ld + k];
    else return M[k * ld + idx];
}

// out[mt] (+)= A[16mt.., 0:16KT] * B, where B (16KT x 16) is given as KT acc
// tiles in registers (PERM map).  A is in LDS, element (i,k) at A[i*lda+k]
// (!A_STRIDED) or A[k*lda+i] (A_STRIDED).  LOWER: A is block lower
// triangular (tiles above the diagonal are zero and need not be multiplied).
template <typename T, int MT, int KT, bool LOWER, bool A_STRIDED>
__device__ __forceinline__ void mm_acc_b(f32x4 (&out)[MT], const T *A, int lda,
                                         const f32x4 (&Bacc)[KT])
{
    const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    if constexpr (is_bf16<T>) {
#pragma unroll
        for (int s = 0; s < (KT + 1) / 2; ++s) {
            const bool two = (2 * s + 1 < KT);
            const bf16x8 b = cat(to_bf16x4(Bacc[2 * s]), two ? to_bf16x4(Bacc[2 * s + 1])
                                                              : to_bf16x4(zero4()));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (LOWER && 2 * s > mt) continue;
                const bf16x4 a1 = run4_lds<A_STRIDED>(A, lda, 16 * mt, 32 * s + 4 * g);
                const bf16x4 a2 = two ? run4_lds<A_STRIDED>(A, lda, 16 * mt, 32 * s + 16 + 4 * g)
                                      : to_bf16x4(zero4());
                out[mt] = mma(cat(a1, a2), b, out[mt]);
            }
        }
    } else if constexpr (!A_STRIDED) {
        // each lane's four k values of a tile are one 16-byte read
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if (LOWER && kt > mt) continue;
                    const float a = one<A_STRIDED>(A, lda, 16 * mt + l16, 16 * kt + 4 * g + r);
                    out[mt] = mma(a, Bacc[kt][r], out[mt]);
                }
            }
        }
    } else {
        // A^T-shaped operand: a lane's values for one k sit in one row, 16
        // floats apart across the MT output tiles, one scalar read each.  The
        // reads of step s + 1 (one k for every tile) are issued before the
        // MFMAs of step s, so their latency is covered by MFMAs; left to
        // itself, a compiler short of registers waits on every read.
        constexpr int NSTEP = 4 * KT;
        float a[2][MT];
        auto load = [&](int st, float (&d)[MT]) {
            const int kt = st >> 2, r = st & 3;
            const float *row = A + (16 * kt + 4 * g + r) * lda + l16;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                if (!(LOWER && kt > mt)) d[mt] = row[16 * mt];
        };
        load(0, a[0]);
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            if (st + 1 < NSTEP) load(st + 1, a[(st + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            const int kt = st >> 2, r = st & 3;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                if (!(LOWER && kt > mt)) out[mt] = mma(a[st & 1][mt], Bacc[kt][r], out[mt]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Workgroup barrier for LDS traffic only: this wave's LDS accesses complete,
// then every wave arrives.  Unlike __syncthreads it does not wait for the
// wave's global loads and stores, which may stay in flight into later phases
// (the compiler waits for each load where its register is first read).  For
// kernels in which no wave reads global memory that another wave of the
// workgroup wrote.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// acc (+)= A[i0:i0+16, 0:K] * B[0:K, j0:j0+16] with both operands in LDS.
// A element (i,k): A[i*lda+k] or, A_STRIDED, A[k*lda+i].
// B element (k,j): B[j*ldb+k] or, B_STRIDED, B[k*ldb+j].
// K must be a multiple of 16.  klim caps the k range (block-triangular
// operands): only k < klim is multiplied; it is a multiple of 16 (bf16: 32,
// or the whole of K).
template <typename T, int K, bool A_STRIDED, bool B_STRIDED>
__device__ __forceinline__ f32x4 mm_lds(f32x4 acc, const T *A, int lda, int i0, const T *B,
                                        int ldb, int j0, int klim = K)
{
    const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
    if constexpr (is_bf16<T>) {
#pragma unroll
        for (int s = 0; s < (K + 31) / 32; ++s) {
            if (32 * s >= klim) break;
            // NAT map.  K = 16: lane groups 2, 3 of the 32-wide k-block lie past
            // K; they read an in-range block (every lane takes part in the
            // transposing read, which exchanges data across its lane group)
            // and zero it afterwards.
            const int k = 32 * s + 8 * g;
            const bool in = k < K;
            const int kr = in ? k : k - 16;
            bf16x8 a = cat(run4_lds<A_STRIDED>(A, lda, i0, kr), run4_lds<A_STRIDED>(A, lda, i0, kr + 4));
            bf16x8 b = cat(run4_lds<B_STRIDED>(B, ldb, j0, kr), run4_lds<B_STRIDED>(B, ldb, j0, kr + 4));
            const bf16x8 z = cat(to_bf16x4(zero4()), to_bf16x4(zero4()));
            a = in ? a : z;
            b = in ? b : z;
            acc = mma(a, b, acc);
        }
    } else {
        // k in 16-wide blocks (klim a multiple of 16).  In block kb the MFMA
        // of step r contracts k = 16 kb + 4 g + r over the lane groups g: a
        // permutation of the block's k, the same for both operands, which
        // puts a lane's four values of a row-major operand side by side.
        // The reads of block kb + 2 are issued before the MFMAs of block kb,
        // so LDS latency is covered by MFMAs instead of stalling each one.
        constexpr int NB = K / 16;
        const int nb = (klim < K ? klim : K) / 16;
        float a[3][4], b[3][4];
        auto load = [&](int kb, float (&av)[4], float (&bv)[4]) {
            const int k0 = 16 * kb + 4 * g;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                av[r] = one<A_STRIDED>(A, lda, i0 + l16, k0 + r);
                bv[r] = one<B_STRIDED>(B, ldb, j0 + l16, k0 + r);
            }
        };
        if (nb > 0) load(0, a[0], b[0]);
        if (nb > 1) load(1, a[1], b[1]);
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
            if (kb >= nb) break;
            if (kb + 2 < nb) load(kb + 2, a[(kb + 2) % 3], b[(kb + 2) % 3]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc = mma(a[kb % 3][r], b[kb % 3][r], acc);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    return acc;
}

// A ROWS x COLS tile of a chunk (COLS contiguous elements per row in global
// memory) held in the registers of the NT threads of a workgroup, 16 bytes per
// thread per step, so that every load of the tile is in flight at once and can
// be issued a chunk ahead of its use.  Rows >= valid are read from row
// valid - 1 (always inside the tensor) and written to LDS as zeros.
template <typename T, int ROWS, int COLS, int NT>
struct TileRegs {
    static constexpr int V = 16 / sizeof(T);
    static_assert(COLS % V == 0, "tile width must be a multiple of 16 bytes");
    static constexpr int VPR = COLS / V;
    static constexpr int N = ROWS * VPR;
    static constexpr int PER = (N + NT - 1) / NT;
    static constexpr bool EXACT = N % NT == 0;
    uint4 r[PER];

    __device__ __forceinline__ void load(const T *g, long g_ld, int valid)
    {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int idx = (int)threadIdx.x + j * NT;
            const int row = min(idx / VPR, valid - 1), cv = idx % VPR;
            if (EXACT || idx < N)
                r[j] = *reinterpret_cast<const uint4 *>(g + (long)row * g_ld + cv * V);
        }
    }

    __device__ __forceinline__ void store(T *s, int s_ld, int valid) const
    {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int idx = (int)threadIdx.x + j * NT;
            const int row = idx / VPR, cv = idx % VPR;
            const unsigned m = row < valid ? ~0u : 0u;
            const uint4 x = make_uint4(r[j].x & m, r[j].y & m, r[j].z & m, r[j].w & m);
            if (EXACT || idx < N) *reinterpret_cast<uint4 *>(s + row * s_ld + cv * V) = x;
        }
    }

    // The same tile widened to fp32 in LDS (s_ld a multiple of 4), rows >=
    // valid as zeros.
    __device__ __forceinline__ void store_f32(float *s, int s_ld, int valid) const
    {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int idx = (int)threadIdx.x + j * NT;
            const int row = idx / VPR, cv = idx % VPR;
            if (EXACT || idx < N) {
                const T *e = reinterpret_cast<const T *>(&r[j]);
                float *d = s + row * s_ld + cv * V;
#pragma unroll
                for (int i = 0; i < V; i += 4) {
                    const bool ok = row < valid;
                    *reinterpret_cast<float4 *>(d + i) =
                        make_float4(ok ? to_f32(e[i]) : 0.f, ok ? to_f32(e[i + 1]) : 0.f,
                                    ok ? to_f32(e[i + 2]) : 0.f, ok ? to_f32(e[i + 3]) : 0.f);
                }
            }
        }
    }
};

// Rows [0, valid) of a ROWS x COLS tile of T in LDS (row stride s_ld, 16-byte
// aligned rows) copied to global memory with 16-byte stores.
template <typename T, int ROWS, int COLS, int NT>
__device__ __forceinline__ void store_rows_t(T *g, long g_ld, const T *s, int s_ld, int valid)
{
    constexpr int V = 16 / sizeof(T), VPR = COLS / V, N = ROWS * VPR;
#pragma unroll
    for (int j = 0; j < (N + NT - 1) / NT; ++j) {
        const int idx = (int)threadIdx.x + j * NT;
        const int row = idx / VPR, cv = idx % VPR;
        if ((N % NT == 0 || idx < N) && row < valid)
            *reinterpret_cast<uint4 *>(g + row * g_ld + cv * V) =
                *reinterpret_cast<const uint4 *>(s + row * s_ld + cv * V);
    }
}

// Rows [0, valid) of a ROWS x COLS fp32 tile in LDS (row stride s_ld, a
// multiple of 4) written to global memory as T with 16-byte non-temporal
// stores (final outputs, not read again by the writer).
template <typename T, int ROWS, int COLS, int NT>
__device__ __forceinline__ void store_rows(T *g, long g_ld, const float *s, int s_ld, int valid)
{
    constexpr int V = 16 / sizeof(T), VPR = COLS / V, N = ROWS * VPR;
#pragma unroll
    for (int j = 0; j < (N + NT - 1) / NT; ++j) {
        const int idx = (int)threadIdx.x + j * NT;
        const int row = idx / VPR, cv = idx % VPR;
        if ((N % NT == 0 || idx < N) && row < valid) {
            const float *src = s + row * s_ld + cv * V;
            uint4 out;
            T *o = reinterpret_cast<T *>(&out);
#pragma unroll
            for (int i = 0; i < V; i += 4) {
                const float4 x = *reinterpret_cast<const float4 *>(src + i);
                o[i] = from_f32<T>(x.x);
                o[i + 1] = from_f32<T>(x.y);
                o[i + 2] = from_f32<T>(x.z);
                o[i + 3] = from_f32<T>(x.w);
            }
            typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, out),
                                        reinterpret_cast<u32x4_t *>(g + row * g_ld + cv * V));
        }
    }
}

// alpha from beta and lambda ("Exact Flow Linear Attention: Exact Solution
// from Continuous-Time Dynamics", Technical Summary, Methodology 3):
// (1 - e^{-beta lambda}) / lambda = beta phi(x), x = beta lambda,
// phi(x) = (1 - e^{-x}) / x = sum_{n>=0} (-x)^n / (n+1)!, phi(0) = 1 -- the
// lambda -> 0 limit alpha = beta.  |x| < 1/2: beta times phi's series to
// n = 9 (the rest is below 3e-11 relative); otherwise 1 - e^{-x} has no
// cancellation and is divided by lambda.  Both are formed and one selected.
__device__ __forceinline__ float efla_alpha(float beta, float lambda)
{
    const float x = beta * lambda, nx = -x;
    constexpr float c[10] = {1.f,           1.f / 2,        1.f / 6,         1.f / 24,
                             1.f / 120,     1.f / 720,      1.f / 5040,      1.f / 40320,
                             1.f / 362880,  1.f / 3628800};
    float p = c[9];
#pragma unroll
    for (int n = 8; n >= 0; --n) p = fmaf(p, nx, c[n]);
    const float e = __builtin_amdgcn_exp2f(nx * 1.44269504088896341f);   // e^{-x}
    const float direct = (1.f - e) * __builtin_amdgcn_rcpf(lambda);
    return fabsf(x) < 0.5f ? beta * p : direct;
}

// alpha under the chosen update: the exact flow's, or beta itself for the
// explicit Euler step of the same ODE (the delta rule the pages compare
// against, Technical Summary, Problem Statement).
__device__ __forceinline__ float update_alpha(int euler, float beta, float lambda)
{
    return euler ? beta : efla_alpha(beta, lambda);
}

// Packed sequences: sequence n of a head spans tokens [packed_begin,
// packed_end) of its L-token axis; offsets out of [0, L] (or a decreasing
// pair) are clamped, so a bad offset shortens or empties a sequence but never
// reaches past the tensor.
__device__ __forceinline__ int packed_begin(const int *cu, int n, int L)
{
    return min(max(cu[n], 0), L);
}
__device__ __forceinline__ int packed_end(const int *cu, int n, int L)
{
    return min(max(cu[n + 1], packed_begin(cu, n, L)), L);
}

// Workgroup -> (sequence, tile) map that keeps the NTILE tiles of one
// sequence on one XCD.  Consecutive workgroup ids are dispatched round-robin
// over the 8 XCDs, so ids x, x+8, x+16, ... share an XCD and its L2.
__device__ __forceinline__ void xcd_map(int bid, int nblocks, int ntile, int &seq, int &tile)
{
    int lin = bid;
    if ((nblocks & 7) == 0) {
        const int per = nblocks >> 3;
        lin = (bid & 7) * per + (bid >> 3);
    }
    seq = lin / ntile;
    tile = lin - seq * ntile;
}

// The same with consecutive units on consecutive XCDs (each unit's ntile
// workgroups still on one XCD): when units carry uneven work (packed
// sequences of varying length), a run of long ones spreads over all XCDs
// instead of landing on one.
__device__ __forceinline__ void xcd_map_rr(int bid, int nblocks, int ntile, int &unit, int &tile)
{
    const int units = nblocks / ntile;
    if (units * ntile == nblocks && (units & 7) == 0) {
        const int x = bid & 7, m = bid >> 3;   // XCD, and the workgroup's place on it
        unit = 8 * (m / ntile) + x;
        tile = m - (m / ntile) * ntile;
    } else {
        unit = bid / ntile;
        tile = bid - unit * ntile;
    }
}

}  // namespace efla
