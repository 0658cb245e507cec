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
