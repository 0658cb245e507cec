"""efla_forward_noalloc (the allocation-free forward) against efla_forward_update
(the same forward with a caller workspace), through the C ABI: two calls in
a row on one device, the second with a smaller input, on the staged and the
segmented paths (whose intermediates live in the library's fixed scratch) and
the fused path (which needs none).  The two entries run the same kernels on
the same inputs, so the outputs must be identical; both are also checked
against the fp64 oracle."""
import pytest
import torch

from delta_rule_sequence_alpha_amd import _lib
import efla_workloads as wl
import oracle
from tests._parity import TOL, dev, note, rel_err

pytestmark = pytest.mark.gpu

PATHS = {"staged": _lib.EFLA_PATH_STAGED, "segmented": _lib.EFLA_PATH_SEGMENTED,
         "fused": _lib.EFLA_PATH_FUSED}

# (path, workload recipe, first shape, second shape (smaller)): (B, H, L, d, C)
CASES = [
    ("staged", "long-stiff-f32", (2, 3, 500, 64, 32), (1, 2, 100, 64, 32)),
    ("staged", "lm1.3b-bf16", (1, 4, 64 * 6 + 40, 128, 64), (1, 2, 70, 128, 64)),
    ("segmented", "long-stiff-f32", (1, 2, 64 * 24 + 9, 128, 64), (1, 2, 64 * 20, 128, 64)),
    ("fused", "lm1.3b-bf16", (1, 4, 64 * 6 + 40, 128, 64), (1, 2, 70, 128, 64)),
]


def _call(fn_name, path, w, q, k, v, beta, S0):
    B, H, L, dk, dv, C = w.B, w.H, w.L, w.d_k, w.d_v, w.chunk
    dt = _lib.EFLA_BF16 if w.dtype == "bf16" else _lib.EFLA_F32
    o = torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device)
    S_L = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    p = lambda x: None if x is None else x.data_ptr()  # noqa: E731
    sp = torch.cuda.current_stream().cuda_stream
    if fn_name == "noalloc":
        st = _lib.efla_forward_noalloc(p(q), p(k), p(v), p(beta), p(S0), p(o), p(S_L), B, H, L,
                                       dk, dv, C, dt, PATHS[path], _lib.EFLA_EXACT, sp)
    else:
        need = _lib.efla_forward_workspace_size_ex(B, H, L, dk, dv, C, dt, PATHS[path])
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        st = _lib.efla_forward_update(p(q), p(k), p(v), p(beta), p(S0), p(o), p(S_L), B, H, L,
                                      dk, dv, C, dt, p(ws), need, PATHS[path], _lib.EFLA_EXACT,
                                      sp)
    assert st == _lib.EFLA_OK, _lib.status_string(st)
    return o, S_L


@pytest.mark.parametrize("path,recipe,first,second", CASES)
def test_noalloc_matches_workspace_entry(path, recipe, first, second):
    for seed, (B, H, L, d, C) in enumerate((first, second)):
        w = wl.FORWARD_WORKLOADS[recipe].with_(B=B, H=H, L=L, d_k=d, d_v=d, chunk=C)
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        need = _lib.efla_forward_workspace_size_ex(B, H, L, d, d, C,
                                                   _lib.EFLA_BF16 if w.dtype == "bf16"
                                                   else _lib.EFLA_F32, PATHS[path])
        assert need <= _lib.NOALLOC_SCRATCH_BYTES
        note(f"noalloc {path} {w.name} B={B} H={H} L={L} d={d} C={C} (call {seed + 1})")
        q, k, v, beta, S0 = wl.forward_inputs(w, seed=40 + seed)
        qd, kd, vd, bd, s0d = dev(q, k, v, beta, S0)
        o_n, S_n = _call("noalloc", path, w, qd, kd, vd, bd, s0d)
        o_w, S_w = _call("workspace", path, w, qd, kd, vd, bd, s0d)
        torch.cuda.synchronize()
        assert o_n.dtype == dt
        assert torch.equal(o_n, o_w) and torch.equal(S_n, S_w)
        o_r, S_r = oracle.forward(q, k, v, beta, S0)
        eo, es = rel_err(o_n, o_r), rel_err(S_n, S_r)
        print(f"  err o={eo:.3e} S_L={es:.3e}", flush=True)
        assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


def test_noalloc_auto_keeps_fused_when_scratch_too_small():
    """bf16, few long sequences: AUTO would take the segmented scan, whose
    intermediates (168 MB here) exceed the scratch array; the allocation-free
    entry then runs the fused kernel, bit for bit as the workspace entry does
    on that path."""
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(B=1, H=8, L=32768)
    need = _lib.efla_forward_workspace_size_ex(1, 8, 32768, 128, 128, 64, _lib.EFLA_BF16,
                                               _lib.EFLA_PATH_AUTO)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    note("noalloc auto fallback to fused, B=1 H=8 L=32768 bf16")
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=45)
    qd, kd, vd, bd, s0d = dev(q, k, v, beta, S0)
    p = lambda x: x.data_ptr()  # noqa: E731
    sp = torch.cuda.current_stream().cuda_stream
    outs = []
    for fused in (False, True):
        o = torch.empty((1, 8, 32768, 128), dtype=torch.bfloat16, device="cuda")
        S_L = torch.empty((1, 8, 128, 128), dtype=torch.float32, device="cuda")
        if fused:
            st = _lib.efla_forward_update(p(qd), p(kd), p(vd), p(bd), p(s0d), p(o), p(S_L), 1, 8,
                                          32768, 128, 128, 64, _lib.EFLA_BF16, None, 0,
                                          _lib.EFLA_PATH_FUSED, _lib.EFLA_EXACT, sp)
        else:
            st = _lib.efla_forward_noalloc(p(qd), p(kd), p(vd), p(bd), p(s0d), p(o), p(S_L), 1, 8,
                                           32768, 128, 128, 64, _lib.EFLA_BF16,
                                           _lib.EFLA_PATH_AUTO, _lib.EFLA_EXACT, sp)
        assert st == _lib.EFLA_OK, _lib.status_string(st)
        outs.append((o, S_L))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    sl = (slice(0, 1), slice(5, 6))
    o_r, S_r = oracle.forward(q[sl], k[sl], v[sl], beta[sl], S0[sl])
    assert rel_err(outs[0][0][sl], o_r) <= TOL["bf16"] and rel_err(outs[0][1][sl], S_r) <= TOL["bf16"]
