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
    // waves per workgroup: the fp32 workgroup is alone on its CU (LDS), so it
    // brings eight waves, two per SIMD; bf16 workgroups fit two per CU at four
    static constexpr int NW = is_bf16<T> ? 4 : 8, NT = 64 * NW;
    static constexpr int PADE = is_bf16<T> ? 8 : 4;   // 16 bytes of row padding
    static constexpr int LDK = DK + PADE, LDV = DV + PADE;
    static constexpr int LDG = C + 1;                  // fp32, scalar access only
    // T (fp32): rows 16-byte aligned, so that a lane's four consecutive k of
    // the A operand of W = T K and U = T V are one 16-byte read
    static constexpr int LDT = C + 4;
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
    static constexpr size_t offTb = offT + sizeof(float) * C * LDT;
    // A = tril(Q K^T) is staged in LDS (rows 16-byte aligned) and written out
    // with 16-byte stores: bf16 in T's bf16 copy, which is only filled after
    // A has been written out, fp32 in a buffer of its own at the same offset
    static constexpr int LDAQ = is_bf16<T> ? LDTB : C + 4;
    static constexpr size_t offAq = offTb;
    static constexpr size_t offA = offTb + (is_bf16<T> ? sizeof(T) * C * LDTB
                                                       : sizeof(float) * C * LDAQ);
    static constexpr size_t bytes = offA + sizeof(float) * C;
};

// Chunk `id` of the launch.  Fixed length: id = bh * nchunks + c is chunk c
// of sequence bh, whose L tokens start at bh * L; A is stored per chunk,
// [BH][nchunks][C][C].  Packed (cu_chunks != NULL): the tensors are [H, L, d]
// with N sequences per head back to back, sequence n at tokens [cu[n],
// cu[n+1]) of its head, and chunks restart at each sequence's first token.
// cu_chunks[n] counts the chunks of the sequences before n; id = h * nchunks
// + i is chunk i - cu_chunks[n] of the sequence n holding the i-th chunk, and
// ids past the last chunk of a head are not chunks (false).  A is then stored
// by token, row r of a chunk at token row tok0 + r of [H, L, C], and only the
// chunk's valid rows.
template <typename T, int C>
struct UtChunk {
    long tok0;
    int valid;
    T *aq;
};

template <typename T, int C>
__device__ __forceinline__ bool ut_locate(int id, int L, int nchunks, const int *cu,
                                          const int *cu_chunks, int N, T *aqk, UtChunk<T, C> &x)
{
    if (!cu_chunks) {
        const int bh = id / nchunks, c = id - bh * nchunks;
        x.tok0 = (long)bh * L + (long)c * C;
        x.valid = min(C, L - c * C);
        x.aq = aqk + ((long)bh * nchunks + c) * C * C;
        return true;
    }
    const int h = id / nchunks, i = id - h * nchunks;
    if (i >= cu_chunks[N]) return false;
    int lo = 0, hi = N;   // last n with cu_chunks[n] <= i
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu_chunks[mid] <= i) lo = mid; else hi = mid;
    }
    const int t0 = packed_begin(cu, lo, L), t1 = packed_end(cu, lo, L);
    const int c = i - cu_chunks[lo];
    x.tok0 = (long)h * L + t0 + (long)c * C;
    x.valid = min(C, t1 - t0 - c * C);
    x.aq = aqk + x.tok0 * C;
    return true;
}

// Tile t of the tiles on and below the diagonal of a block matrix, row by
// row: t = it (it + 1) / 2 + jt, jt <= it.
__device__ __forceinline__ void lower_tile(int t, int &it, int &jt)
{
    it = 0;
    while (t > it) {
        t -= it + 1;
        ++it;
    }
    jt = t;
}

// The first chunk id >= id (stepping by `stride`) that is a chunk, or an id
// >= total.
template <typename T, int C>
__device__ __forceinline__ long ut_next(long id, int stride, int total, int L, int nchunks,
                                       const int *cu, const int *cu_chunks, int N, T *aqk,
                                       UtChunk<T, C> &x)
{
    while (id < total && !ut_locate<T, C>((int)id, L, nchunks, cu, cu_chunks, N, aqk, x))
        id += stride;
    return id;
}

// Persistent: workgroup b takes chunks b, b + gridDim.x, ... of the `total`
// ids, and the next chunk's K and Q tiles (and, once this chunk has staged
// its V tile, the next V tile) are loaded into registers while this chunk is
// computed, so the loads' latency is not exposed once per chunk.
// alpha == NULL: the coefficients are formed here from beta (and euler), with
// lambda_r = k_r . k_r the diagonal of the chunk's Gram matrix; alpha_out and
// lambda_out, if not NULL, receive alpha_r and lambda_r of every valid token.
template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__((UtLayout<T, DK, DV, C>::NT)) void ut_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ alpha, T *__restrict__ w, T *__restrict__ u, T *__restrict__ aqk,
    int L, int nchunks, const int *__restrict__ cu, const int *__restrict__ cu_chunks, int N,
    int total, const float *__restrict__ beta, int euler, float *__restrict__ alpha_out,
    float *__restrict__ lambda_out)
{
    using Lay = UtLayout<T, DK, DV, C>;
    constexpr int NW = Lay::NW, NT = 64 * NW, MC = C / 16;
    constexpr bool BF = is_bf16<T>;
    extern __shared__ __align__(16) char smem[];
    T *sK = reinterpret_cast<T *>(smem + Lay::offK);
    T *sQ = reinterpret_cast<T *>(smem + Lay::offQ);
    T *sV = reinterpret_cast<T *>(smem + Lay::offV);
    float *sG = reinterpret_cast<float *>(smem + Lay::offG);
    float *sT = reinterpret_cast<float *>(smem + Lay::offT);
    T *sTb = reinterpret_cast<T *>(smem + Lay::offTb);
    float *sAl = reinterpret_cast<float *>(smem + Lay::offA);
    T *sAq = reinterpret_cast<T *>(smem + Lay::offAq);

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
    const bool packed = cu_chunks != nullptr;
    const int stride = gridDim.x;

    // T's blocks above the diagonal are never written in the loop: zero them
    // once (the bf16 copy of T reads them; the first chunk's barrier orders it)
    for (int i = threadIdx.x; i < C * Lay::LDT; i += NT) sT[i] = 0.f;
    // likewise the tiles of A's staging above the diagonal, which no chunk
    // writes (in bf16 the copy of T rewrites them, with T's zeros)
    for (int i = threadIdx.x; i < C * Lay::LDAQ; i += NT) sAq[i] = from_f32<T>(0.f);

    UtChunk<T, C> cur, nxt;
    long id = ut_next<T, C>(blockIdx.x, stride, total, L, nchunks, cu, cu_chunks, N, aqk, cur);
    TileRegs<T, C, DK, NT> tk, tq;
    TileRegs<T, C, DV, NT> tv;
    if (id < total) {
        tk.load(k + cur.tok0 * DK, DK, cur.valid);
        tq.load(q + cur.tok0 * DK, DK, cur.valid);
        tv.load(v + cur.tok0 * DV, DV, cur.valid);
    }
    while (id < total) {   // uniform over the workgroup
        const long tok0 = cur.tok0;
        const int valid = cur.valid;
        T *const aq = cur.aq;
        const long nid =
            ut_next<T, C>(id + stride, stride, total, L, nchunks, cu, cu_chunks, N, aqk, nxt);

        tk.store(sK, Lay::LDK, valid);
        tq.store(sQ, Lay::LDK, valid);
        float be = 0.f;   // alpha from beta: token `lane` of the chunk, wave 0
        if (alpha) {
            for (int i = threadIdx.x; i < C; i += NT) sAl[i] = (i < valid) ? alpha[tok0 + i] : 0.f;
        } else if (wv == 0 && lane < valid) {
            be = beta[tok0 + lane];
        }
        __syncthreads();
        if (nid < total) {   // the next chunk's K and Q fly while this one is computed
            tk.load(k + nxt.tok0 * DK, DK, nxt.valid);
            tq.load(q + nxt.tok0 * DK, DK, nxt.valid);
        }

        // The tiles on and below the diagonal: of G = K K^T (fp32 into LDS) and
        // of A = tril(Q K^T) (staged in LDS).  The first phase takes every
        // Gram tile and the first NA tiles of A, NA evening out the count
        // over the four SIMDs (wave w runs on SIMD w mod 4).
        constexpr int NLOW = MC * (MC + 1) / 2;
        constexpr int NA = (4 - NLOW % 4) % 4 < NLOW ? (4 - NLOW % 4) % 4 : NLOW;
        auto a_tile = [&](int t) {
            int it, jt;
            lower_tile(t, it, jt);
            const f32x4 acc = mm_lds<T, DK, false, false>(zero4(), sQ, Lay::LDK, 16 * it, sK,
                                                          Lay::LDK, 16 * jt);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * it + 4 * g + r, col = 16 * jt + l16;
                sAq[row * Lay::LDAQ + col] = from_f32<T>(col <= row ? acc[r] : 0.f);
            }
        };
        for (int t = wv; t < NLOW + NA; t += NW) {
            if (t < NLOW) {
                int it, jt;
                lower_tile(t, it, jt);
                const f32x4 acc = mm_lds<T, DK, false, false>(zero4(), sK, Lay::LDK, 16 * it, sK,
                                                              Lay::LDK, 16 * jt);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sG[(16 * it + 4 * g + r) * Lay::LDG + 16 * jt + l16] = acc[r];
            } else {
                a_tile(t - NLOW);
            }
        }
        __syncthreads();

        if (wv == 0) {
            // Wave 0: alpha of token `lane` from beta and the Gram diagonal, then
            // the diagonal 16x16 blocks of T by forward substitution, lane group b
            // handling block b, lane l16 column l16 of it (LDS keeps one wave's
            // accesses in order).
            if (!alpha && lane < C) {
                const float lam = sG[lane * Lay::LDG + lane];
                const float al = lane < valid ? update_alpha(euler, be, lam) : 0.f;
                sAl[lane] = al;
                if (alpha_out && lane < valid) {
                    alpha_out[tok0 + lane] = al;
                    lambda_out[tok0 + lane] = lam;
                }
            }
            if (g < MC) {
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
                for (int i = 0; i < 16; ++i) sT[(b0 + i) * Lay::LDT + b0 + j] = t[i];
            }
        } else {
            // The other waves meanwhile: the remaining tiles of A
            for (int t = NA + wv - 1; t < NLOW; t += NW - 1) a_tile(t);
        }
        __syncthreads();

        // Blocks below the diagonal (fp32 MFMA): wave j solves column block j
        // from the top, T_ij = -T_ii sum_{m=j}^{i-1} G_im T_mj for i = j+1 ..
        // MC-1, right-looking: once T_mj is known, its term is added to the
        // sums of every later block row at once, so those MFMAs are
        // independent of each other and only T_ii (sum) waits on the chain.
        // A solved block stays in registers in the accumulator layout (rows
        // 4g + r of column l16), which is the B operand of the next products
        // when a lane's four MFMAs take k = 4g + r.  A column needs only its
        // own blocks and the diagonal ones, so the columns proceed side by
        // side with no barrier between block rows.  The waves not needed for
        // it write A out of its staging with 16-byte stores (every row;
        // packed, the chunk's valid rows only).
        tv.store(sV, Lay::LDV, valid);   // A = tril(Q K^T) is done with Q
        if (wv < MC - 1) {
            constexpr int NB = MC > 1 ? MC - 1 : 1;
            const int bj = wv, nb = MC - 1 - bj;   // blocks below the diagonal in column bj
            // G_{bj+1+d, bj+m} (m <= d), row l16, k = 4g + r: every one read up front
            float gv[NB][NB][4];
#pragma unroll
            for (int d = 0; d < MC - 1; ++d)
#pragma unroll
                for (int m = 0; m <= d; ++m) {
                    const int bi = min(bj + 1 + d, MC - 1), bm = min(bj + m, MC - 1);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        gv[d][m][r] = sG[(16 * bi + l16) * Lay::LDG + 16 * bm + 4 * g + r];
                }
            f32x4 tb, p[NB];
#pragma unroll
            for (int r = 0; r < 4; ++r) tb[r] = sT[(16 * bj + 4 * g + r) * Lay::LDT + 16 * bj + l16];
#pragma unroll
            for (int d = 0; d < MC - 1; ++d) p[d] = zero4();
#pragma unroll
            for (int m = 0; m < MC - 1; ++m) {
                if (m >= nb) break;
                // tb = T_{bj+m, bj}: its term in every later block row
#pragma unroll
                for (int d = m; d < MC - 1; ++d)
                    if (d < nb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) p[d] = mma(gv[d][m][r], tb[r], p[d]);
                // the sum of block row bn is complete: T_{bn, bj} = -T_{bn, bn} p
                const int bn = bj + m + 1;
                const f32x4 tnn = *reinterpret_cast<const f32x4 *>(
                    sT + (16 * bn + l16) * Lay::LDT + 16 * bn + 4 * g);
                f32x4 x = zero4();
#pragma unroll
                for (int r = 0; r < 4; ++r) x = mma(tnn[r], p[m][r], x);
                tb = -x;
#pragma unroll
                for (int r = 0; r < 4; ++r) sT[(16 * bn + 4 * g + r) * Lay::LDT + 16 * bj + l16] = tb[r];
            }
        } else {
            constexpr int VA = 16 / (int)sizeof(T), VPR = C / VA, T0 = 64 * (MC - 1);
            const int arows = packed ? valid : C;
            for (int idx = (int)threadIdx.x - T0; idx < C * VPR; idx += NT - T0) {
                const int row = idx / VPR, cv = idx - row * VPR;
                if (row < arows)
                    *reinterpret_cast<uint4 *>(aq + row * C + cv * VA) =
                        *reinterpret_cast<const uint4 *>(sAq + row * Lay::LDAQ + cv * VA);
            }
        }
        __syncthreads();

        const T *sTop = nullptr;   // T as the MFMA A operand
        int ldTop = 0;
        if constexpr (BF) {
            // four elements per step: a 16-byte read, an 8-byte write
            for (int i = threadIdx.x; i < C * C / 4; i += NT) {
                const int r = i / (C / 4), cc = 4 * (i - r * (C / 4));
                *reinterpret_cast<bf16x4 *>(sTb + r * Lay::LDTB + cc) =
                    to_bf16x4(*reinterpret_cast<const f32x4 *>(sT + r * Lay::LDT + cc));
            }
            sTop = sTb;
            ldTop = Lay::LDTB;
            __syncthreads();
        } else {
            sTop = reinterpret_cast<const T *>(sT);
            ldTop = Lay::LDT;
        }
        // the next V tile flies during the products (the barrier above would
        // have waited for it)
        if (nid < total) tv.load(v + nxt.tok0 * DV, DV, nxt.valid);

        // W = T K and U = T V (T lower triangular: k range of row tile mt is
        // [0, 16mt+16)), each staged in LDS over the operand it no longer
        // needs (W over K, U over V) and written with 16-byte stores.  fp32
        // forms both in one phase and holds them in registers until every
        // read of K and V is done; bf16, whose four-wave workgroups share a CU
        // in pairs, keeps to its register budget with a phase for each.
        constexpr int NTK = DK / 16, NTV = DV / 16;
        constexpr int WPW = (MC * NTK + NW - 1) / NW, UPW = (MC * NTV + NW - 1) / NW;   // per wave
        constexpr bool ONE_PHASE = !BF;
        auto w_tiles = [&](f32x4 (&acc)[WPW]) {
#pragma unroll
            for (int j = 0; j < WPW; ++j) {
                const int t = wv + NW * j, mt = t / NTK, nt = t - mt * NTK;
                if (t < MC * NTK)
                    acc[j] = mm_lds<T, C, false, true>(zero4(), sTop, ldTop, 16 * mt, sK,
                                                       Lay::LDK, 16 * nt, 16 * mt + 16);
            }
        };
        auto u_tiles = [&](f32x4 (&acc)[UPW]) {
#pragma unroll
            for (int j = 0; j < UPW; ++j) {
                const int t = wv + NW * j, mt = t / NTV, nt = t - mt * NTV;
                if (t < MC * NTV)
                    acc[j] = mm_lds<T, C, false, true>(zero4(), sTop, ldTop, 16 * mt, sV,
                                                       Lay::LDV, 16 * nt, 16 * mt + 16);
            }
        };
        auto stage_w = [&](const f32x4 (&acc)[WPW]) {
#pragma unroll
            for (int j = 0; j < WPW; ++j) {
                const int t = wv + NW * j, mt = t / NTK, nt = t - mt * NTK;
                if (t < MC * NTK)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sK[(16 * mt + 4 * g + r) * Lay::LDK + 16 * nt + l16] = from_f32<T>(acc[j][r]);
            }
        };
        auto stage_u = [&](const f32x4 (&acc)[UPW]) {
#pragma unroll
            for (int j = 0; j < UPW; ++j) {
                const int t = wv + NW * j, mt = t / NTV, nt = t - mt * NTV;
                if (t < MC * NTV)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sV[(16 * mt + 4 * g + r) * Lay::LDV + 16 * nt + l16] = from_f32<T>(acc[j][r]);
            }
        };
        if constexpr (ONE_PHASE) {
            f32x4 accW[WPW], accU[UPW];
            w_tiles(accW);
            u_tiles(accU);
            __syncthreads();   // every read of K and V is done
            stage_w(accW);
            stage_u(accU);
        } else {
            f32x4 accW[WPW];
            w_tiles(accW);
            __syncthreads();   // every read of K is done
            stage_w(accW);
            f32x4 accU[UPW];
            u_tiles(accU);
            __syncthreads();   // every read of V is done; W is staged
            stage_u(accU);
        }
        __syncthreads();
        store_rows_t<T, C, DK, NT>(w + tok0 * DK, DK, sK, Lay::LDK, valid);
        store_rows_t<T, C, DV, NT>(u + tok0 * DV, DV, sV, Lay::LDV, valid);
        __syncthreads();   // the staged W and U are read before the next chunk's tiles land
        id = nid;
        cur = nxt;
    }
}

// cu_chunks[n] = chunks of packed sequences 0 .. n-1 (n = 0 .. N), capped
// at cap.  One workgroup: each thread sums a run of sequences, the 256 run
// totals are scanned in LDS, and each thread writes its run's offsets.
__global__ __launch_bounds__(256) void packed_chunks_kernel(const int *__restrict__ cu, int N,
                                                            int L, int C, int cap,
                                                            int *__restrict__ cu_chunks)
{
    __shared__ long long part[256];
    const int t = threadIdx.x, per = (N + 255) / 256;
    const int n0 = min(N, t * per), n1 = min(N, n0 + per);
    auto chunks = [&](int n) {
        return (long long)(packed_end(cu, n, L) - packed_begin(cu, n, L) + C - 1) / C;
    };
    long long sum = 0;
    for (int n = n0; n < n1; ++n) sum += chunks(n);
    part[t] = sum;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const long long x = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += x;
        __syncthreads();
    }
    long long run = t ? part[t - 1] : 0;
    for (int n = n0; n < n1; ++n) {
        cu_chunks[n] = (int)min(run, (long long)cap);
        run += chunks(n);
    }
    if (t == 255) cu_chunks[N] = (int)min(part[255], (long long)cap);
}

hipError_t dispatch_packed_chunks(const int *cu, int N, int L, int chunk, int *cu_chunks,
                                  hipStream_t st)
{
    const int cap = (L + chunk - 1) / chunk + N;
    hipLaunchKernelGGL(packed_chunks_kernel, dim3(1), dim3(256), 0, st, cu, N, L, chunk, cap,
                       cu_chunks);
    return hipGetLastError();
}

constexpr size_t kLdsPerCu = 160 * 1024;   // gfx950

template <typename T, int DK, int DV, int C>
hipError_t launch_ut(const void *q, const void *k, const void *v, const float *alpha, void *w,
                     void *u, void *aqk, int BH, int L, const int *cu, const int *cu_chunks, int N,
                     int H, const float *beta, bool euler, float *alpha_out, float *lambda_out,
                     hipStream_t st)
{
    using Lay = UtLayout<T, DK, DV, C>;
    const int nchunks = (L + C - 1) / C;
    if (BH == 0 || nchunks == 0) return hipSuccess;
    const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&ut_kernel<T, DK, DV, C>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
    if (attr != hipSuccess) return attr;
    // packed: per head, at most one chunk more per sequence than whole chunks
    const int per = cu_chunks ? nchunks + N : nchunks;
    const long total = (long)(cu_chunks ? H : BH) * per;
    // as many workgroups as the CUs hold at once (LDS-bound), each looping
    // over chunks
    const long resident = 256L * (long)(kLdsPerCu / Lay::bytes > 0 ? kLdsPerCu / Lay::bytes : 1);
    const long grid = total < resident ? total : resident;
    hipLaunchKernelGGL((ut_kernel<T, DK, DV, C>), dim3((unsigned)grid), dim3(Lay::NT), Lay::bytes,
                       st, static_cast<const T *>(q), static_cast<const T *>(k),
                       static_cast<const T *>(v), alpha, static_cast<T *>(w),
                       static_cast<T *>(u), static_cast<T *>(aqk), L, per, cu, cu_chunks, N,
                       (int)total, beta, (int)euler, alpha_out, lambda_out);
    return hipGetLastError();
}

hipError_t dispatch_ut(bool bf16, int dk, int dv, int chunk, const void *q, const void *k,
                       const void *v, const float *alpha, void *w, void *u, void *aqk, int BH,
                       int L, hipStream_t st, const int *cu, const int *cu_chunks, int N, int H,
                       const float *beta, bool euler, float *alpha_out, float *lambda_out)
{
#define CASE(DKV, DVV, CC)                                                                      \
    if (dk == DKV && dv == DVV && chunk == CC)                                                  \
        return bf16 ? launch_ut<__bf16, DKV, DVV, CC>(q, k, v, alpha, w, u, aqk, BH, L, cu,     \
                                                      cu_chunks, N, H, beta, euler, alpha_out, \
                                                      lambda_out, st)                          \
                    : launch_ut<float, DKV, DVV, CC>(q, k, v, alpha, w, u, aqk, BH, L, cu,      \
                                                     cu_chunks, N, H, beta, euler, alpha_out,  \
                                                     lambda_out, st);
    EFLA_SHAPE_CASES(CASE)
#undef CASE
    return hipErrorInvalidValue;
}

}  // namespace efla
