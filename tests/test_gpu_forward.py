"""Parity of efla_forward with the fp64 oracle: the five workloads (reduced
sizes element by element, full sizes on sampled heads), ragged tails, empty
inputs, aliasing, degenerate tokens, determinism and structural properties."""
import numpy as np
import pytest
import torch

import delta_rule_sequence_alpha_amd as efla
import efla_workloads as wl
import oracle
from tests._parity import TOL, dev, note, rel_err

pytestmark = pytest.mark.gpu

PATHS = ["staged", "fused"]


def _skip_unsupported(path, dtype):
    if path == "fused" and dtype != "bf16":
        pytest.skip("the fused kernel takes bf16 inputs; fp32 runs the staged kernels")


def _run(w, path, seed=0, S0_override=None):
    _skip_unsupported(path, w.dtype)
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=seed)
    if S0_override is not None:
        S0 = S0_override
    qd, kd, vd, bd, s0d = dev(q, k, v, beta, S0)
    o, S_L = efla.forward(qd, kd, vd, bd, s0d, chunk=w.chunk, path=path)
    torch.cuda.synchronize()
    return (q, k, v, beta, S0), o, S_L


def _check(w, inputs, o, S_L, heads=None):
    q, k, v, beta, S0 = inputs
    tol = TOL[w.dtype]
    if heads is None:
        o_r, S_r = oracle.forward(q, k, v, beta, S0)
        eo, es = rel_err(o, o_r), rel_err(S_L, S_r)
    else:
        eo = es = 0.0
        for b, h in heads:
            sl = (slice(b, b + 1), slice(h, h + 1))
            o_r, S_r = oracle.forward(q[sl], k[sl], v[sl], beta[sl], None if S0 is None else S0[sl])
            eo = max(eo, rel_err(o[sl], o_r))
            es = max(es, rel_err(S_L[sl], S_r))
    print(f"  err o={eo:.3e} S_L={es:.3e} (gate {tol:g})", flush=True)
    assert eo <= tol and es <= tol
    return eo, es


# --- the five workloads ------------------------------------------------------

@pytest.mark.parametrize("path", PATHS)
def test_tiny_f32(path):
    w = wl.FORWARD_WORKLOADS["tiny-f32"]
    note(f"forward {w.name} {path}")
    inputs, o, S_L = _run(w, path)
    _check(w, inputs, o, S_L)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name,B,H,L", [("lm340m-bf16", 2, 3, 64 * 5 + 17),
                                        ("lm1.3b-bf16", 1, 4, 64 * 6 + 40),
                                        ("long-stiff-f32", 1, 3, 64 * 9 + 5)])
def test_workload_recipes_reduced(path, name, B, H, L):
    w = wl.FORWARD_WORKLOADS[name].with_(B=B, H=H, L=L)
    note(f"forward {name} reduced B={B} H={H} L={L} {path}")
    inputs, o, S_L = _run(w, path, seed=1)
    _check(w, inputs, o, S_L)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name,heads", [("lm340m-bf16", [(0, 0), (3, 5), (7, 7)]),
                                        ("lm1.3b-bf16", [(0, 0), (1, 9), (3, 15)]),
                                        ("long-stiff-f32", [(0, 0), (0, 11)])])
def test_workload_full_size_sampled_heads(path, name, heads):
    w = wl.FORWARD_WORKLOADS[name]
    note(f"forward {name} full size {path}")
    inputs, o, S_L = _run(w, path)
    assert torch.isfinite(o).all() and torch.isfinite(S_L).all()
    _check(w, inputs, o, S_L, heads=heads)


# --- shapes, tails and edges -------------------------------------------------

@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,chunk,L", [(16, 16, 16, 1), (16, 16, 16, 15), (32, 32, 32, 96),
                                           (64, 64, 64, 63), (128, 64, 64, 129), (64, 128, 32, 100),
                                           (16, 128, 16, 50), (128, 16, 64, 70), (32, 16, 16, 33)])
def test_shapes_and_ragged_tails(path, dtype, dk, dv, chunk, L):
    w = wl.FORWARD_WORKLOADS["long-stiff-f32"].with_(B=2, H=1, L=L, d_k=dk, d_v=dv, chunk=chunk,
                                                     dtype=dtype)
    note(f"forward shape {dtype} dk={dk} dv={dv} C={chunk} L={L} {path}")
    S0 = torch.randn(2, 1, dk, dv, generator=torch.Generator().manual_seed(L)) * 0.1
    inputs, o, S_L = _run(w, path, seed=L, S0_override=S0)
    _check(w, inputs, o, S_L)


@pytest.mark.parametrize("path", PATHS)
def test_empty_sequence_copies_state(path):
    note(f"forward L=0 {path}")
    S0 = torch.randn(2, 3, 32, 16).cuda()
    e = torch.empty(2, 3, 0, 32, device="cuda", dtype=torch.bfloat16)
    ev = torch.empty(2, 3, 0, 16, device="cuda", dtype=torch.bfloat16)
    o, S_L = efla.forward(e, e, ev, torch.empty(2, 3, 0, device="cuda"), S0, chunk=16, path=path)
    o2, S_L2 = efla.forward(e, e, ev, torch.empty(2, 3, 0, device="cuda"), None, chunk=16,
                            path=path)
    torch.cuda.synchronize()
    assert o.shape == (2, 3, 0, 16)
    assert torch.equal(S_L, S0)
    assert torch.count_nonzero(S_L2) == 0


@pytest.mark.parametrize("path", PATHS)
def test_state_aliasing_in_place(path):
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(B=1, H=2, L=200)
    note(f"forward aliasing S0 == S_L {path}")
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=3)
    qd, kd, vd, bd, sd = dev(q, k, v, beta, S0)
    o, S_L = efla.forward(qd, kd, vd, bd, sd, chunk=64, path=path, S_L=sd)
    torch.cuda.synchronize()
    assert S_L.data_ptr() == sd.data_ptr()
    _check(w, (q, k, v, beta, S0), o, S_L)


def _segmented_splits(w):
    """True when the segmented path's plan splits this shape (its workspace
    then holds segment maps beyond the staged path's)."""
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    args = (w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, dt)
    return efla.workspace_size(*args, "segmented") > efla.workspace_size(*args, "staged")


# (path, dtype, L, beta = 0 span in head 0, k = 0 span in head 1).  The
# segmented case is long enough to be split, and its spans cross segments.
DEGENERATE_CASES = [("fused", "bf16", 48, (10, 30), (5, 40)),
                    ("staged", "bf16", 48, (10, 30), (5, 40)),
                    ("staged", "f32", 48, (10, 30), (5, 40)),
                    ("segmented", "f32", 16 * 24, (60, 200), (100, 300))]


@pytest.mark.parametrize("path,dtype,L,zb,zk", DEGENERATE_CASES)
def test_degenerate_tokens_are_identity(path, dtype, L, zb, zk):
    """beta = 0 or k = 0 tokens leave the state unchanged: alpha k k^T = 0 and
    alpha k v^T = 0 (Methodology 3), so over a beta = 0 span o_t = S^T q_t
    with S frozen at the state entering the span."""
    w = wl.FORWARD_WORKLOADS["tiny-f32"].with_(H=2, L=L, dtype=dtype)
    if path == "segmented":
        assert _segmented_splits(w)
    note(f"forward degenerate tokens {path} {dtype} L={L}")
    q, k, v, beta, _ = wl.forward_inputs(w, seed=4)
    beta[:, 0, zb[0]:zb[1]] = 0.0
    k[:, 1, zk[0]:zk[1]] = 0.0
    inputs = (q, k, v, beta, None)
    qd, kd, vd, bd = dev(q, k, v, beta)
    o, S_L = efla.forward(qd, kd, vd, bd, None, chunk=16, path=path)
    torch.cuda.synchronize()
    _check(w, inputs, o, S_L)
    t0, t1 = zb
    _, S_in = oracle.forward(q[:, :, :t0], k[:, :, :t0], v[:, :, :t0], beta[:, :, :t0])
    frozen = np.einsum("bhij,bhti->bhtj", S_in[:, :1], q[:, :1, t0:t1].double().numpy())
    assert rel_err(o[:, :1, t0:t1], frozen) <= TOL[w.dtype]


@pytest.mark.parametrize("path", PATHS)
def test_nan_stays_in_its_head(path):
    w = wl.FORWARD_WORKLOADS["lm340m-bf16"].with_(B=1, H=4, L=130)
    note(f"forward NaN isolation {path}")
    q, k, v, beta, _ = wl.forward_inputs(w, seed=5)
    clean = efla.forward(*dev(q, k, v, beta), None, chunk=64, path=path)
    vb = v.clone()
    vb[0, 2, 7, 3] = float("nan")
    dirty = efla.forward(*dev(q, k, vb, beta), None, chunk=64, path=path)
    torch.cuda.synchronize()
    for h in (0, 1, 3):
        assert torch.equal(clean[0][:, h], dirty[0][:, h])
        assert torch.equal(clean[1][:, h], dirty[1][:, h])
    assert torch.isnan(dirty[1][:, 2]).any()


@pytest.mark.parametrize("path", PATHS)
def test_deterministic_and_column_permutation(path):
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(B=1, H=2, L=256)
    note(f"forward determinism + column permutation {path}")
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=6)
    a = efla.forward(*dev(q, k, v, beta, S0), chunk=64, path=path)
    b = efla.forward(*dev(q, k, v, beta, S0), chunk=64, path=path)
    perm = torch.randperm(128, generator=torch.Generator().manual_seed(0))
    c = efla.forward(*dev(q, k, v[..., perm].contiguous(), beta, S0[..., perm].contiguous()),
                     chunk=64, path=path)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(c[0], a[0][..., perm]) and torch.equal(c[1], a[1][..., perm])


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("t0", [64, 100])
def test_split_and_resume(path, t0):
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(H=2, L=256, dtype="f32" if path == "staged" else "bf16")
    _skip_unsupported(path, w.dtype)
    note(f"forward split/resume t0={t0} {path}")
    q, k, v, beta, _ = wl.forward_inputs(w, seed=7)
    qd, kd, vd, bd = dev(q, k, v, beta)
    o, S = efla.forward(qd, kd, vd, bd, None, chunk=64, path=path)
    oa, Sa = efla.forward(*[x[:, :, :t0].contiguous() for x in (qd, kd, vd, bd)], None, chunk=64,
                          path=path)
    ob, Sb = efla.forward(*[x[:, :, t0:].contiguous() for x in (qd, kd, vd, bd)], Sa, chunk=64,
                          path=path)
    torch.cuda.synchronize()
    o_r, S_r = oracle.forward(q, k, v, beta)
    tol = TOL[w.dtype]
    assert rel_err(torch.cat([oa, ob], dim=2), o_r) <= tol
    assert rel_err(Sb, S_r) <= tol
    assert rel_err(S, S_r) <= tol


# (path, L, t0): the stiff fp32 recipe, split at t0 and resumed from the
# first part's state.  The segmented sizes are long enough that the whole
# sequence and both parts are each split into segments.
STIFF_SPLITS = [("staged", 64 * 6 + 9, 64 * 3), ("staged", 64 * 6 + 9, 100),
                ("segmented", 64 * 40, 64 * 20 + 17)]


@pytest.mark.parametrize("path,L,t0", STIFF_SPLITS)
def test_split_and_resume_stiff_f32(path, L, t0):
    """A sequence split at t0, the second part starting from the first part's
    final state, equals the whole (the recurrence is sequential in S,
    Methodology 3), on the stiff recipe (beta lambda up to 5e4) in fp32."""
    w = wl.FORWARD_WORKLOADS["long-stiff-f32"].with_(B=1, H=2, L=L)
    if path == "segmented":
        for part in (w, w.with_(L=t0), w.with_(L=L - t0)):
            assert _segmented_splits(part), part
    note(f"forward stiff split/resume {path} L={L} t0={t0}")
    q, k, v, beta, _ = wl.forward_inputs(w, seed=8)
    qd, kd, vd, bd = dev(q, k, v, beta)
    o, S = efla.forward(qd, kd, vd, bd, None, chunk=64, path=path)
    oa, Sa = efla.forward(*[x[:, :, :t0].contiguous() for x in (qd, kd, vd, bd)], None, chunk=64,
                          path=path)
    ob, Sb = efla.forward(*[x[:, :, t0:].contiguous() for x in (qd, kd, vd, bd)], Sa, chunk=64,
                          path=path)
    torch.cuda.synchronize()
    o_r, S_r = oracle.forward(q, k, v, beta)
    tol = TOL["f32"]
    e = (rel_err(torch.cat([oa, ob], dim=2), o_r), rel_err(Sb, S_r), rel_err(o, o_r),
         rel_err(S, S_r))
    print(f"  err split o={e[0]:.3e} S={e[1]:.3e} whole o={e[2]:.3e} S={e[3]:.3e}", flush=True)
    assert max(e) <= tol


@pytest.mark.parametrize("path,dtype", [("fused", "bf16"), ("staged", "bf16"), ("staged", "f32"),
                                        ("segmented", "f32")])
def test_affine_in_state_and_values(path, dtype):
    """With q, k, beta fixed the outputs are linear in (S0, V) jointly (the
    update and readout are linear in S and v).  Scaling both by 2 is exact in
    binary floating point, so o(2 S0, 2 V) = 2 o(S0, V) bit for bit; and for
    fp32 inputs o(S0 + S0', V + V') = o(S0, V) + o(S0', V') within fp32
    rounding."""
    L = 64 * 24 + 9 if path == "segmented" else 64 * 3 + 29
    w = wl.FORWARD_WORKLOADS["long-stiff-f32"].with_(B=1, H=2, L=L, dtype=dtype)
    note(f"forward affinity {path} {dtype} L={L}")
    q, k, v, beta, _ = wl.forward_inputs(w, seed=47)
    g = torch.Generator().manual_seed(47)
    S0 = torch.randn(1, 2, w.d_k, w.d_v, generator=g) * 0.1
    v2 = (torch.randn(v.shape, generator=g)).to(v.dtype)
    S02 = torch.randn(1, 2, w.d_k, w.d_v, generator=g) * 0.1
    run = lambda vv, ss: efla.forward(*dev(q, k, vv, beta, ss), chunk=w.chunk, path=path)  # noqa: E731
    o1, s1 = run(v, S0)
    o2, s2 = run((2 * v.float()).to(v.dtype), 2 * S0)
    torch.cuda.synchronize()
    assert torch.equal(o2, 2 * o1) and torch.equal(s2, 2 * s1)
    if dtype == "f32":
        o3, s3 = run(v2, S02)
        o4, s4 = run(v + v2, S0 + S02)
        torch.cuda.synchronize()
        assert rel_err(o4, (o1 + o3).double().cpu().numpy()) <= 1e-5
        assert rel_err(s4, (s1 + s3).double().cpu().numpy()) <= 1e-5
