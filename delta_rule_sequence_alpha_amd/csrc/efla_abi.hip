// Host side of the C ABI declared in include/efla.h: argument validation (no
// HIP call before it passes), workspace sizing, and kernel launches on the
// caller's stream.
#include <stdint.h>

#include <atomic>

#include "efla.h"
#include "efla_launch.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool chunk_ok(int c) { return c == 16 || c == 32 || c == 64; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t esize(efla_dtype_t dt) { return dt == EFLA_BF16 ? 2 : 4; }

// Shape checks common to the chunked entry points.
efla_status_t check_shape(int B, int H, int L, int dk, int dv, int chunk, efla_dtype_t dt)
{
    if (dt != EFLA_F32 && dt != EFLA_BF16) return EFLA_ERR_INVALID_ARG;
    if (B < 0 || H < 0 || L < 0 || dk <= 0 || dv <= 0 || chunk <= 0) return EFLA_ERR_INVALID_ARG;
    if (!dim_ok(dk) || !dim_ok(dv) || !chunk_ok(chunk)) return EFLA_ERR_UNSUPPORTED;
    // grid sizes and element offsets must fit their types
    const long long bh = (long long)B * H;
    const long long nchunks = ((long long)L + chunk - 1) / chunk;
    if (bh * nchunks > INT32_MAX || bh * 8 > INT32_MAX) return EFLA_ERR_UNSUPPORTED;
    if (bh * (long long)L * (dk > dv ? dk : dv) > (1LL << 46)) return EFLA_ERR_UNSUPPORTED;
    return EFLA_OK;
}

// Segments of the segmented scan: enough (sequence, segment, column tile)
// workgroups in its summary pass for ~2 per CU of the 256, with at least 4
// chunks per segment.  G = 1 means splitting does not pay.  wide: the
// forward's fp32 passes at d_k = d_v = 128, whose workgroups take 128
// columns (8 waves) instead of 64.
struct SegPlan {
    int G, seg_chunks;
};

SegPlan seg_plan(long long BH, int L, int dk, int dv, int chunk, bool wide = false)
{
    const int nchunks = (L + chunk - 1) / chunk;
    const int dmin = dk < dv ? dk : dv;
    const int tv = wide && dmin >= 128 ? 128 : dmin >= 64 ? 64 : dmin;   // columns per summary workgroup
    const long long tiles = BH * ((dk + dv) / tv);
    long long G = (512 + tiles - 1) / (tiles > 0 ? tiles : 1);
    if (G > nchunks / 4) G = nchunks / 4;
    // it costs about three scans' work: only worth it with many segments on
    // a GPU the plain scan leaves mostly idle
    if (G < 4 || BH * ((dv + 63) / 64) >= 128) G = 1;
    SegPlan p;
    p.seg_chunks = (int)((nchunks + G - 1) / G);
    p.G = p.seg_chunks > 0 ? (nchunks + p.seg_chunks - 1) / p.seg_chunks : 1;
    return p;
}

// Staged / segmented forward workspace: W, U and A (input dtype; the UT
// transform forms alpha itself), and for G > 1 segments the segment maps and
// entry states (fp32).
struct StagedWs {
    size_t w, u, aqk, R, P, Sin, total;
};

StagedWs staged_ws(int B, int H, int L, int dk, int dv, int chunk, efla_dtype_t dt, int G)
{
    const size_t n = (size_t)B * H * L;
    const size_t nch = (size_t)B * H * ((L + chunk - 1) / chunk);
    const size_t segs = (size_t)B * H * G;
    StagedWs s;
    s.w = 0;
    s.u = s.w + align_up(n * dk * esize(dt));
    s.aqk = s.u + align_up(n * dv * esize(dt));
    s.R = s.aqk + align_up(nch * chunk * chunk * esize(dt));
    s.total = s.R;
    s.P = s.Sin = s.R;
    if (G > 1) {   // the segmented scan's maps and entry states (fp32)
        s.P = s.R + align_up(segs * dk * dv * sizeof(float));
        s.Sin = s.P + align_up(segs * dk * dk * sizeof(float));
        s.total = s.Sin + align_up(segs * dk * dv * sizeof(float));
    }
    return s;
}

// Packed-sequence (varlen) staged workspace: W, U over every token of the H
// heads, A by token ([H, T, chunk]), the chunk offsets of the sequences
// (int32 [N+1]) and, for G > 1 segments per sequence, the segment maps and
// entry states (fp32).
struct VarlenWs {
    size_t w, u, aqk, cuc, R, P, Sin, total;
};

VarlenWs varlen_ws(int N, int H, int T, int dk, int dv, int chunk, efla_dtype_t dt, int G)
{
    const size_t n = (size_t)H * T;
    const size_t segs = (size_t)N * H * G;
    VarlenWs s;
    s.w = 0;
    s.u = s.w + align_up(n * dk * esize(dt));
    s.aqk = s.u + align_up(n * dv * esize(dt));
    s.cuc = s.aqk + align_up(n * chunk * esize(dt));
    s.R = s.cuc + align_up(((size_t)N + 1) * sizeof(int));
    s.total = s.P = s.Sin = s.R;
    if (G > 1) {
        s.P = s.R + align_up(segs * dk * dv * sizeof(float));
        s.Sin = s.P + align_up(segs * dk * dk * sizeof(float));
        s.total = s.Sin + align_up(segs * dk * dv * sizeof(float));
    }
    return s;
}

// Shape checks of the packed entry points: the tensors are [H, T, d] (one
// "batch" of H rows of T tokens) and N * H sequences; the UT transform's grid
// has at most ceil(T / chunk) + N chunks per head.
efla_status_t check_varlen(int N, int H, int T, int dk, int dv, int chunk, efla_dtype_t dt)
{
    const efla_status_t s = check_shape(1, H, T, dk, dv, chunk, dt);
    if (s != EFLA_OK) return s;
    if (N < 0) return EFLA_ERR_INVALID_ARG;
    const long long NH = (long long)N * H;
    if (NH * 8 > INT32_MAX) return EFLA_ERR_UNSUPPORTED;
    if ((long long)H * (((long long)T + chunk - 1) / chunk + N) > INT32_MAX)
        return EFLA_ERR_UNSUPPORTED;
    return EFLA_OK;
}

efla_path_t auto_path(efla_dtype_t dt, long long BH, int L, int dk, int dv, int chunk);

int varlen_G(efla_path_t p, int N, int H, int T, int dk, int dv, int chunk, bool wide);

// The packed path.  AUTO for bf16 as for fixed lengths (auto_path).  For
// fp32 the host knows no lengths and the longest sequence bounds the plain
// scan, so it takes the segmented scan whenever the plain scan's workgroups
// (N H d_v / 64) are fewer than the CUs and a sequence as long as the whole
// token axis would be split.
efla_path_t resolve_varlen_path(efla_path_t p, efla_dtype_t dt, int N, int H, int T, int dk,
                                int dv, int chunk)
{
    if (p != EFLA_PATH_AUTO) return p;
    const long long NH = (long long)N * H;
    if (efla::fused_supported(dt == EFLA_BF16, dk, dv, chunk))
        return auto_path(dt, NH, T, dk, dv, chunk);
    const bool few = NH * ((dv + 63) / 64) < 256;
    return few && varlen_G(EFLA_PATH_SEGMENTED, N, H, T, dk, dv, chunk, dt == EFLA_F32) > 1
               ? EFLA_PATH_SEGMENTED
               : EFLA_PATH_STAGED;
}

// Segments per packed sequence: planned for one sequence per head holding the
// whole token axis (the longest a sequence can be; shorter ones leave
// segments empty), capped at 4096 (sequence, head, segment) units in all so
// the maps stay modest (each unit's are 2 d_k d_v + d_k^2 floats).
int varlen_G(efla_path_t p, int N, int H, int T, int dk, int dv, int chunk, bool wide)
{
    if (p != EFLA_PATH_SEGMENTED) return 1;
    const long long units = (long long)N * H > 0 ? (long long)N * H : 1;
    long long G = seg_plan(H, T, dk, dv, chunk, wide).G;
    if (G * units > 4096) G = 4096 / units > 1 ? 4096 / units : 1;
    return (int)G;
}

// Backward workspace: the forward's coefficient and UT-transform outputs,
// plus every chunk's entry state, dS_out and dE (in the input dtype), and for
// G > 1 segments the segment maps and boundary states (fp32) that the two
// segmented scans use one after the other.
struct BackwardWs {
    size_t alpha, lambda, w, u, aqk, states, dSout, dE, R, P, Sin, total;
};

BackwardWs backward_ws(int B, int H, int L, int dk, int dv, int chunk, efla_dtype_t dt, int G)
{
    const size_t n = (size_t)B * H * L;
    const size_t nch = (size_t)B * H * ((L + chunk - 1) / chunk);
    const size_t segs = (size_t)B * H * G;
    BackwardWs s;
    s.alpha = 0;
    s.lambda = s.alpha + align_up(n * sizeof(float));
    s.w = s.lambda + align_up(n * sizeof(float));
    s.u = s.w + align_up(n * dk * esize(dt));
    s.aqk = s.u + align_up(n * dv * esize(dt));
    s.states = s.aqk + align_up(nch * chunk * chunk * esize(dt));
    s.dSout = s.states + align_up(nch * dk * dv * esize(dt));
    s.dE = s.dSout + align_up(nch * dk * dv * esize(dt));
    s.R = s.dE + align_up(nch * chunk * dv * esize(dt));
    s.total = s.P = s.Sin = s.R;
    if (G > 1) {
        s.P = s.R + align_up(segs * dk * dv * sizeof(float));
        s.Sin = s.P + align_up(segs * dk * dk * sizeof(float));
        s.total = s.Sin + align_up(segs * dk * dv * sizeof(float));
    }
    return s;
}

// AUTO: the fused kernel where it exists (bf16 inputs), unless it would run
// so few workgroups (one per sequence and 32 state columns) that most CUs
// idle while the segmented scan splits the sequences: at d = 128, C = 64 the
// fused kernel took 0.66 ms and the segmented path 0.41 ms for 1 x 8 heads x
// 32768 tokens (32 workgroups), against 1.32 and 1.52 ms for 1 x 16 x 65536
// (64 workgroups).  Otherwise (fp32) the segmented scan when it has more
// than one segment per sequence, else the staged one.
constexpr long long kFusedFewWorkgroups = 32;

efla_path_t auto_path(efla_dtype_t dt, long long BH, int L, int dk, int dv, int chunk)
{
    const int G = seg_plan(BH, L, dk, dv, chunk, dt == EFLA_F32).G;
    if (efla::fused_supported(dt == EFLA_BF16, dk, dv, chunk)) {
        const long long fused_wgs = BH * ((dv + 31) / 32);
        return fused_wgs <= kFusedFewWorkgroups && G > 1 ? EFLA_PATH_SEGMENTED : EFLA_PATH_FUSED;
    }
    return G > 1 ? EFLA_PATH_SEGMENTED : EFLA_PATH_STAGED;
}

efla_path_t resolve_path(efla_path_t p, efla_dtype_t dt, int B, int H, int L, int dk, int dv,
                         int chunk)
{
    if (p != EFLA_PATH_AUTO) return p;
    return auto_path(dt, (long long)B * H, L, dk, dv, chunk);
}

int plan_G(efla_path_t p, int B, int H, int L, int dk, int dv, int chunk, bool wide)
{
    return p == EFLA_PATH_SEGMENTED ? seg_plan((long long)B * H, L, dk, dv, chunk, wide).G : 1;
}

// Launch configuration: every field 0 (or no struct) is the built-in choice.
// The backward's two scans default to 4-wave (64-column) workgroups.
// Unsegmented they share one launch, whose workgroups then fill the CUs
// (lm1.3b-bf16: 270 us for both at 4 waves, 297 at 2; run one after the
// other they took 197 + 232 us at 2 waves).  Segmented scans have
// workgroups to spare (long-stiff-f32: 1.5 vs 2.6 ms per state-scan pass
// at 4 vs 2 waves).
efla_launch_config_t config_of(const efla_launch_config_t *c)
{
    efla_launch_config_t r{0, 0, 0};
    if (c) r = *c;
    if (r.bwd_scan_waves == 0) r.bwd_scan_waves = 4;
    return r;
}

bool config_ok(const efla_launch_config_t *c)
{
    if (!c) return true;
    auto w124 = [](int n) { return n == 0 || n == 1 || n == 2 || n == 4; };
    return (c->fused_scan_waves == 0 || c->fused_scan_waves == 1 || c->fused_scan_waves == 2) &&
           (w124(c->scan_waves) || c->scan_waves == 8) && w124(c->bwd_scan_waves);
}

efla_status_t hip_status(hipError_t e) { return e == hipSuccess ? EFLA_OK : EFLA_ERR_HIP; }

}  // namespace

extern "C" {

const char *efla_status_string(efla_status_t s)
{
    switch (s) {
    case EFLA_OK: return "EFLA_OK";
    case EFLA_ERR_INVALID_ARG: return "EFLA_ERR_INVALID_ARG";
    case EFLA_ERR_UNSUPPORTED: return "EFLA_ERR_UNSUPPORTED";
    case EFLA_ERR_WORKSPACE: return "EFLA_ERR_WORKSPACE";
    case EFLA_ERR_HIP: return "EFLA_ERR_HIP";
    }
    return "EFLA_ERR_UNKNOWN";
}

efla_path_t efla_forward_path(int B, int H, int L, int dk, int dv, int chunk, efla_dtype_t dt)
{
    if (check_shape(B, H, L, dk, dv, chunk, dt) != EFLA_OK) return EFLA_PATH_AUTO;
    return resolve_path(EFLA_PATH_AUTO, dt, B, H, L, dk, dv, chunk);
}

size_t efla_forward_workspace_size_ex(int B, int H, int L, int dk, int dv, int chunk,
                                      efla_dtype_t dt, efla_path_t path)
{
    if (check_shape(B, H, L, dk, dv, chunk, dt) != EFLA_OK) return 0;
    path = resolve_path(path, dt, B, H, L, dk, dv, chunk);
    if (path == EFLA_PATH_STAGED || path == EFLA_PATH_SEGMENTED)
        return staged_ws(B, H, L, dk, dv, chunk, dt, plan_G(path, B, H, L, dk, dv, chunk, dt == EFLA_F32)).total;
    return 0;
}

size_t efla_forward_workspace_size(int B, int H, int L, int dk, int dv, int chunk, efla_dtype_t dt)
{
    return efla_forward_workspace_size_ex(B, H, L, dk, dv, chunk, dt, EFLA_PATH_AUTO);
}

}  // extern "C"

namespace {

// The allocation-free forward's scratch: the staged and segmented paths'
// intermediates, in a fixed device array that the library holds on each
// device it runs on.  Host code never uses the array's name as an address
// (on the host it names a stand-in); the device address is looked up once
// per device, with that device current, and kept.
constexpr size_t kScratchBytes = EFLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];
std::atomic<void *> g_scratch_ptr[kMaxDevices];

hipError_t scratch_address(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

// The forward after the entry point's own argument: intermediates of the
// staged and segmented paths in `workspace`, or (noalloc) in the scratch
// array above, for shapes whose workspace fits in it.
efla_status_t forward_impl(const void *q, const void *k, const void *v, const float *beta,
                           const float *S0, void *o, float *S_L, int B, int H, int L, int dk,
                           int dv, int chunk, efla_dtype_t dt, void *workspace,
                           size_t workspace_bytes, efla_path_t path, efla_update_t update,
                           const efla_launch_config_t *config, bool noalloc, void *stream)
{
    efla_status_t s = check_shape(B, H, L, dk, dv, chunk, dt);
    if (s != EFLA_OK) return s;
    if (update != EFLA_EXACT && update != EFLA_EULER) return EFLA_ERR_INVALID_ARG;
    if (!config_ok(config)) return EFLA_ERR_INVALID_ARG;
    const efla_launch_config_t cfg = config_of(config);
    const bool euler = update == EFLA_EULER;
    if (path != EFLA_PATH_AUTO && path != EFLA_PATH_STAGED && path != EFLA_PATH_FUSED &&
        path != EFLA_PATH_SEGMENTED)
        return EFLA_ERR_INVALID_ARG;
    const bool auto_chosen = path == EFLA_PATH_AUTO;
    path = resolve_path(path, dt, B, H, L, dk, dv, chunk);
    // allocation-free: AUTO keeps to the fused kernel (no intermediates) when
    // the path it would take does not fit in the scratch array
    if (noalloc && auto_chosen && path != EFLA_PATH_FUSED &&
        efla::fused_supported(dt == EFLA_BF16, dk, dv, chunk) &&
        staged_ws(B, H, L, dk, dv, chunk, dt, plan_G(path, B, H, L, dk, dv, chunk, dt == EFLA_F32))
                .total > kScratchBytes)
        path = EFLA_PATH_FUSED;
    const long long BH = (long long)B * H;
    if (BH == 0) return EFLA_OK;
    if (!S_L || !aligned16(S_L) || (S0 && !aligned16(S0))) return EFLA_ERR_INVALID_ARG;
    if (L > 0) {
        if (!q || !k || !v || !beta || !o) return EFLA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(o))
            return EFLA_ERR_INVALID_ARG;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (path == EFLA_PATH_FUSED) {
        if (!efla::fused_supported(dt == EFLA_BF16, dk, dv, chunk)) return EFLA_ERR_UNSUPPORTED;
        if (L == 0) return hip_status(efla::launch_copy_state(S0, S_L, BH * dk * dv, st));
        return hip_status(efla::dispatch_fused(dt == EFLA_BF16, dk, dv, chunk, q, k, v, beta, S0,
                                               o, S_L, (int)BH, L, cfg.fused_scan_waves, euler,
                                               st));
    }
    const SegPlan plan = path == EFLA_PATH_SEGMENTED ? seg_plan(BH, L, dk, dv, chunk, dt == EFLA_F32)
                                                     : SegPlan{1, 0};
    const StagedWs ws = staged_ws(B, H, L, dk, dv, chunk, dt, plan.G);
    if (noalloc && L > 0) {
        if (ws.total > kScratchBytes) return EFLA_ERR_WORKSPACE;
        const hipError_t e = scratch_address(&workspace);
        if (e != hipSuccess) return EFLA_ERR_HIP;
        workspace_bytes = kScratchBytes;
    }
    if (L > 0) {
        if (!workspace || workspace_bytes < ws.total) return EFLA_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return EFLA_ERR_INVALID_ARG;
    }

    if (L == 0) return hip_status(efla::launch_copy_state(S0, S_L, BH * dk * dv, st));

    const bool bf = dt == EFLA_BF16;
    char *base = static_cast<char *>(workspace);
    void *w = base + ws.w, *u = base + ws.u, *aqk = base + ws.aqk;
    hipError_t e = efla::dispatch_ut(bf, dk, dv, chunk, q, k, v, nullptr, w, u, aqk, (int)BH, L,
                                     st, nullptr, nullptr, 0, 1, beta, euler);
    if (e == hipSuccess && plan.G > 1)
        e = efla::dispatch_scan_segmented(bf, dk, dv, chunk, q, k, w, u, aqk, S0, o, S_L, (int)BH, L,
                                          plan.G, plan.seg_chunks,
                                          reinterpret_cast<float *>(base + ws.R),
                                          reinterpret_cast<float *>(base + ws.P),
                                          reinterpret_cast<float *>(base + ws.Sin),
                                          cfg.scan_waves, st);
    else if (e == hipSuccess)
        e = efla::dispatch_scan(bf, dk, dv, chunk, q, k, w, u, aqk, S0, o, S_L, (int)BH, L,
                                cfg.scan_waves, st);
    return hip_status(e);
}

}  // namespace

extern "C" {

efla_status_t efla_forward_config(const void *q, const void *k, const void *v, const float *beta,
                                  const float *S0, void *o, float *S_L, int B, int H, int L,
                                  int dk, int dv, int chunk, efla_dtype_t dt, void *workspace,
                                  size_t workspace_bytes, efla_path_t path, efla_update_t update,
                                  const efla_launch_config_t *config, void *stream)
{
    return forward_impl(q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt, workspace,
                        workspace_bytes, path, update, config, false, stream);
}

efla_status_t efla_forward_noalloc(const void *q, const void *k, const void *v, const float *beta,
                                   const float *S0, void *o, float *S_L, int B, int H, int L,
                                   int dk, int dv, int chunk, efla_dtype_t dt, efla_path_t path,
                                   efla_update_t update, void *stream)
{
    return forward_impl(q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt, nullptr, 0, path,
                        update, nullptr, true, stream);
}

efla_status_t efla_forward_update(const void *q, const void *k, const void *v, const float *beta,
                                  const float *S0, void *o, float *S_L, int B, int H, int L,
                                  int dk, int dv, int chunk, efla_dtype_t dt, void *workspace,
                                  size_t workspace_bytes, efla_path_t path, efla_update_t update,
                                  void *stream)
{
    return efla_forward_config(q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt, workspace,
                               workspace_bytes, path, update, nullptr, stream);
}

size_t efla_forward_varlen_workspace_size(int N, int H, int T, int dk, int dv, int chunk,
                                          efla_dtype_t dt, efla_path_t path)
{
    if (check_varlen(N, H, T, dk, dv, chunk, dt) != EFLA_OK) return 0;
    path = resolve_varlen_path(path, dt, N, H, T, dk, dv, chunk);
    if (path != EFLA_PATH_STAGED && path != EFLA_PATH_SEGMENTED) return 0;
    return varlen_ws(N, H, T, dk, dv, chunk, dt, varlen_G(path, N, H, T, dk, dv, chunk, dt == EFLA_F32)).total;
}

efla_status_t efla_forward_varlen_ex(const void *q, const void *k, const void *v,
                                     const float *beta, const int *cu_seqlens, const float *S0,
                                     void *o, float *S_L, int N, int H, int T, int dk, int dv,
                                     int chunk, efla_dtype_t dt, efla_update_t update,
                                     efla_path_t path, void *workspace, size_t workspace_bytes,
                                     void *stream)
{
    efla_status_t s = check_varlen(N, H, T, dk, dv, chunk, dt);
    if (s != EFLA_OK) return s;
    if (update != EFLA_EXACT && update != EFLA_EULER) return EFLA_ERR_INVALID_ARG;
    if (path != EFLA_PATH_AUTO && path != EFLA_PATH_STAGED && path != EFLA_PATH_FUSED &&
        path != EFLA_PATH_SEGMENTED)
        return EFLA_ERR_INVALID_ARG;
    path = resolve_varlen_path(path, dt, N, H, T, dk, dv, chunk);
    const bool bf = dt == EFLA_BF16, euler = update == EFLA_EULER;
    if (path == EFLA_PATH_FUSED && !efla::fused_supported(bf, dk, dv, chunk))
        return EFLA_ERR_UNSUPPORTED;
    const long long NH = (long long)N * H;
    if (NH == 0) return EFLA_OK;
    if (!cu_seqlens || !S_L || !aligned16(S_L) || (S0 && !aligned16(S0)))
        return EFLA_ERR_INVALID_ARG;
    if (T > 0) {
        if (!q || !k || !v || !beta || !o) return EFLA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(o))
            return EFLA_ERR_INVALID_ARG;
    }
    const int G = varlen_G(path, N, H, T, dk, dv, chunk, dt == EFLA_F32);
    const VarlenWs ws = varlen_ws(N, H, T, dk, dv, chunk, dt, G);
    if (path != EFLA_PATH_FUSED && T > 0) {
        if (!workspace || workspace_bytes < ws.total) return EFLA_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return EFLA_ERR_INVALID_ARG;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (T == 0) return hip_status(efla::launch_copy_state(S0, S_L, NH * dk * dv, st));
    if (path == EFLA_PATH_FUSED)
        return hip_status(efla::dispatch_fused_varlen(bf, dk, dv, chunk, q, k, v, beta, S0, o, S_L,
                                                      (int)NH, T, cu_seqlens, H, 0, euler, st));

    char *base = static_cast<char *>(workspace);
    void *w = base + ws.w, *u = base + ws.u, *aqk = base + ws.aqk;
    int *cuc = reinterpret_cast<int *>(base + ws.cuc);
    hipError_t e = efla::dispatch_packed_chunks(cu_seqlens, N, T, chunk, cuc, st);
    if (e == hipSuccess)
        e = efla::dispatch_ut(bf, dk, dv, chunk, q, k, v, nullptr, w, u, aqk, H, T, st, cu_seqlens,
                              cuc, N, H, beta, euler);
    if (e == hipSuccess && G > 1)
        e = efla::dispatch_scan_segmented(bf, dk, dv, chunk, q, k, w, u, aqk, S0, o, S_L, (int)NH,
                                          T, G, 0, reinterpret_cast<float *>(base + ws.R),
                                          reinterpret_cast<float *>(base + ws.P),
                                          reinterpret_cast<float *>(base + ws.Sin), 0, st,
                                          cu_seqlens, H);
    else if (e == hipSuccess)
        e = efla::dispatch_scan(bf, dk, dv, chunk, q, k, w, u, aqk, S0, o, S_L, (int)NH, T, 0, st,
                                cu_seqlens, H);
    return hip_status(e);
}

efla_status_t efla_forward_varlen(const void *q, const void *k, const void *v, const float *beta,
                                  const int *cu_seqlens, const float *S0, void *o, float *S_L,
                                  int N, int H, int T, int dk, int dv, int chunk, efla_dtype_t dt,
                                  efla_update_t update, void *stream)
{
    return efla_forward_varlen_ex(q, k, v, beta, cu_seqlens, S0, o, S_L, N, H, T, dk, dv, chunk,
                                  dt, update, EFLA_PATH_FUSED, nullptr, 0, stream);
}

efla_status_t efla_forward_ex(const void *q, const void *k, const void *v, const float *beta,
                              const float *S0, void *o, float *S_L, int B, int H, int L, int dk,
                              int dv, int chunk, efla_dtype_t dt, void *workspace,
                              size_t workspace_bytes, efla_path_t path, void *stream)
{
    return efla_forward_update(q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt, workspace,
                               workspace_bytes, path, EFLA_EXACT, stream);
}

efla_status_t efla_forward(const void *q, const void *k, const void *v, const float *beta,
                           const float *S0, void *o, float *S_L, int B, int H, int L, int dk,
                           int dv, int chunk, efla_dtype_t dt, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    return efla_forward_ex(q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt, workspace,
                           workspace_bytes, EFLA_PATH_AUTO, stream);
}

efla_status_t efla_decode_step_update(const void *q, const void *k, const void *v,
                                      const float *beta, float *S, void *o, int N, int H, int dk,
                                      int dv, efla_dtype_t dt, efla_update_t update, void *stream)
{
    if (dt != EFLA_F32 && dt != EFLA_BF16) return EFLA_ERR_INVALID_ARG;
    if (update != EFLA_EXACT && update != EFLA_EULER) return EFLA_ERR_INVALID_ARG;
    if (N < 0 || H < 0 || dk <= 0 || dv <= 0) return EFLA_ERR_INVALID_ARG;
    if (!dim_ok(dk) || !dim_ok(dv)) return EFLA_ERR_UNSUPPORTED;
    const long long NH = (long long)N * H;
    if (NH > INT32_MAX) return EFLA_ERR_UNSUPPORTED;
    if (NH == 0) return EFLA_OK;
    if (!q || !k || !v || !beta || !S || !o) return EFLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(S) ||
        !aligned16(o))
        return EFLA_ERR_INVALID_ARG;
    return hip_status(efla::dispatch_decode(dt == EFLA_BF16, dk, dv, q, k, v, beta, S, o, NH,
                                            update == EFLA_EULER, static_cast<hipStream_t>(stream)));
}

efla_status_t efla_decode_step_indexed(const void *q, const void *k, const void *v,
                                       const float *beta, const int *slots, float *S_pool, void *o,
                                       int *err, int N, int H, int P, int dk, int dv,
                                       efla_dtype_t dt, efla_update_t update, void *stream)
{
    if (dt != EFLA_F32 && dt != EFLA_BF16) return EFLA_ERR_INVALID_ARG;
    if (update != EFLA_EXACT && update != EFLA_EULER) return EFLA_ERR_INVALID_ARG;
    if (N < 0 || H < 0 || P < 0 || dk <= 0 || dv <= 0) return EFLA_ERR_INVALID_ARG;
    if (!dim_ok(dk) || !dim_ok(dv)) return EFLA_ERR_UNSUPPORTED;
    const long long NH = (long long)N * H;
    if (NH > INT32_MAX || (long long)P * H > INT32_MAX) return EFLA_ERR_UNSUPPORTED;
    if (NH == 0) return EFLA_OK;
    if (!q || !k || !v || !beta || !slots || !S_pool || !o) return EFLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(beta) ||
        !aligned16(S_pool) || !aligned16(o))
        return EFLA_ERR_INVALID_ARG;
    return hip_status(efla::dispatch_decode(dt == EFLA_BF16, dk, dv, q, k, v, beta, S_pool, o, NH,
                                            update == EFLA_EULER, static_cast<hipStream_t>(stream),
                                            slots, N, H, P, err));
}

efla_status_t efla_decode_step(const void *q, const void *k, const void *v, const float *beta,
                               float *S, void *o, int N, int H, int dk, int dv, efla_dtype_t dt,
                               void *stream)
{
    return efla_decode_step_update(q, k, v, beta, S, o, N, H, dk, dv, dt, EFLA_EXACT, stream);
}

efla_status_t efla_coefficients_update(const void *k, const float *beta, float *alpha,
                                       float *lambda, long n_tokens, int dk, efla_dtype_t dt,
                                       efla_update_t update, void *stream)
{
    if (dt != EFLA_F32 && dt != EFLA_BF16) return EFLA_ERR_INVALID_ARG;
    if (update != EFLA_EXACT && update != EFLA_EULER) return EFLA_ERR_INVALID_ARG;
    if (n_tokens < 0 || dk <= 0) return EFLA_ERR_INVALID_ARG;
    if (!dim_ok(dk)) return EFLA_ERR_UNSUPPORTED;
    if (n_tokens == 0) return EFLA_OK;
    if ((n_tokens + 255) / 256 > INT32_MAX) return EFLA_ERR_UNSUPPORTED;
    if (!k || !beta || !alpha || !aligned16(k)) return EFLA_ERR_INVALID_ARG;
    return hip_status(efla::dispatch_coef(dt == EFLA_BF16, dk, k, beta, alpha, lambda, n_tokens,
                                          update == EFLA_EULER, static_cast<hipStream_t>(stream)));
}

efla_status_t efla_coefficients(const void *k, const float *beta, float *alpha, float *lambda,
                                long n_tokens, int dk, efla_dtype_t dt, void *stream)
{
    return efla_coefficients_update(k, beta, alpha, lambda, n_tokens, dk, dt, EFLA_EXACT, stream);
}

efla_status_t efla_ut_transform(const void *q, const void *k, const void *v, const float *alpha,
                                void *w, void *u, void *a_qk, int B, int H, int L, int dk, int dv,
                                int chunk, efla_dtype_t dt, void *stream)
{
    efla_status_t s = check_shape(B, H, L, dk, dv, chunk, dt);
    if (s != EFLA_OK) return s;
    const long long BH = (long long)B * H;
    if (BH == 0 || L == 0) return EFLA_OK;
    if (!q || !k || !v || !alpha || !w || !u || !a_qk) return EFLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(w) || !aligned16(u) ||
        !aligned16(a_qk))
        return EFLA_ERR_INVALID_ARG;
    return hip_status(efla::dispatch_ut(dt == EFLA_BF16, dk, dv, chunk, q, k, v, alpha, w, u, a_qk,
                                        (int)BH, L, static_cast<hipStream_t>(stream)));
}

efla_status_t efla_chunk_scan(const void *q, const void *k, const void *w, const void *u,
                              const void *a_qk, const float *S0, void *o, float *S_L, int B, int H,
                              int L, int dk, int dv, int chunk, efla_dtype_t dt, void *stream)
{
    efla_status_t s = check_shape(B, H, L, dk, dv, chunk, dt);
    if (s != EFLA_OK) return s;
    const long long BH = (long long)B * H;
    if (BH == 0) return EFLA_OK;
    if (!S_L || !aligned16(S_L) || (S0 && !aligned16(S0))) return EFLA_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (L == 0) return hip_status(efla::launch_copy_state(S0, S_L, BH * dk * dv, st));
    if (!q || !k || !w || !u || !a_qk || !o) return EFLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(w) || !aligned16(u) || !aligned16(a_qk) ||
        !aligned16(o))
        return EFLA_ERR_INVALID_ARG;
    return hip_status(efla::dispatch_scan(dt == EFLA_BF16, dk, dv, chunk, q, k, w, u, a_qk, S0, o,
                                          S_L, (int)BH, L, 0, st));
}

size_t efla_backward_workspace_size(int B, int H, int L, int dk, int dv, int chunk,
                                    efla_dtype_t dt)
{
    if (check_shape(B, H, L, dk, dv, chunk, dt) != EFLA_OK) return 0;
    if (L == 0 || (long long)B * H == 0) return 0;
    return backward_ws(B, H, L, dk, dv, chunk, dt,
                       seg_plan((long long)B * H, L, dk, dv, chunk).G).total;
}

efla_status_t efla_backward_config(const void *q, const void *k, const void *v, const float *beta,
                                   const float *S0, const void *d_o, const float *dS_L, void *dq,
                                   void *dk_out, void *dv_out, float *dbeta, float *dS0, int B,
                                   int H, int L, int dk, int dv, int chunk, efla_dtype_t dt,
                                   efla_update_t update, const efla_launch_config_t *config,
                                   void *workspace, size_t workspace_bytes, void *stream)
{
    efla_status_t s = check_shape(B, H, L, dk, dv, chunk, dt);
    if (s != EFLA_OK) return s;
    if (update != EFLA_EXACT && update != EFLA_EULER) return EFLA_ERR_INVALID_ARG;
    if (!config_ok(config)) return EFLA_ERR_INVALID_ARG;
    const efla_launch_config_t cfg = config_of(config);
    const bool euler = update == EFLA_EULER;
    const long long BH = (long long)B * H;
    if (BH == 0) return EFLA_OK;
    if ((S0 && !aligned16(S0)) || (dS_L && !aligned16(dS_L)) || (dS0 && !aligned16(dS0)))
        return EFLA_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (L == 0) {   // S_L = S0: dLoss/dS0 = dS_L
        if (!dS0) return EFLA_OK;
        return hip_status(efla::launch_copy_state(dS_L, dS0, BH * dk * dv, st));
    }
    if (!q || !k || !v || !beta || !d_o || !dq || !dk_out || !dv_out || !dbeta)
        return EFLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(d_o) ||
        !aligned16(dq) || !aligned16(dk_out) || !aligned16(dv_out) || !aligned16(dbeta))
        return EFLA_ERR_INVALID_ARG;
    // few long sequences: both scans split over L, as the forward's AUTO path
    const SegPlan plan = seg_plan(BH, L, dk, dv, chunk);
    const BackwardWs ws = backward_ws(B, H, L, dk, dv, chunk, dt, plan.G);
    if (!workspace || workspace_bytes < ws.total) return EFLA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return EFLA_ERR_INVALID_ARG;

    const bool bf = dt == EFLA_BF16;
    char *base = static_cast<char *>(workspace);
    float *alpha = reinterpret_cast<float *>(base + ws.alpha);
    float *lambda = reinterpret_cast<float *>(base + ws.lambda);
    void *w = base + ws.w, *u = base + ws.u, *aqk = base + ws.aqk;
    void *states = base + ws.states, *dSout = base + ws.dSout, *dE = base + ws.dE;
    float *R = reinterpret_cast<float *>(base + ws.R), *P = reinterpret_cast<float *>(base + ws.P);
    float *Sin = reinterpret_cast<float *>(base + ws.Sin);
    // the UT transform forms alpha and lambda (the Gram diagonal) and keeps them
    // for the gradient kernel
    hipError_t e = efla::dispatch_ut(bf, dk, dv, chunk, q, k, v, nullptr, w, u, aqk, (int)BH, L,
                                     st, nullptr, nullptr, 0, 1, beta, euler, alpha, lambda);
    const int nw = cfg.bwd_scan_waves;
    if (e == hipSuccess && plan.G == 1) {   // the two scans are independent: one launch
        e = efla::dispatch_scan_pair(bf, dk, dv, chunk, q, k, w, u, aqk, S0, states, d_o, dS_L,
                                     dSout, dE, dS0, (int)BH, L, nw, st);
    } else if (e == hipSuccess) {           // segmented: one after the other (shared scratch)
        e = efla::dispatch_scan_states(bf, dk, dv, chunk, q, k, w, u, aqk, S0, states, (int)BH, L,
                                       nw, plan.G, plan.seg_chunks, R, P, Sin, st);
        if (e == hipSuccess)
            e = efla::dispatch_rscan(bf, dk, dv, chunk, q, k, w, aqk, d_o, dS_L, dSout, dE, dS0,
                                     (int)BH, L, nw, plan.G, plan.seg_chunks, R, P, Sin, st);
    }
    if (e == hipSuccess)
        e = efla::dispatch_grad(bf, dk, dv, chunk, q, k, v, d_o, beta, alpha, lambda, states,
                                dSout, dE, dq, dk_out, dv_out, dbeta, (int)BH, L, euler, st);
    return hip_status(e);
}

efla_status_t efla_backward(const void *q, const void *k, const void *v, const float *beta,
                            const float *S0, const void *d_o, const float *dS_L, void *dq,
                            void *dk_out, void *dv_out, float *dbeta, float *dS0, int B, int H,
                            int L, int dk, int dv, int chunk, efla_dtype_t dt,
                            efla_update_t update, void *workspace, size_t workspace_bytes,
                            void *stream)
{
    return efla_backward_config(q, k, v, beta, S0, d_o, dS_L, dq, dk_out, dv_out, dbeta, dS0, B,
                                H, L, dk, dv, chunk, dt, update, nullptr, workspace,
                                workspace_bytes, stream);
}

}  // extern "C"
