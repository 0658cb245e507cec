"""Parity of efla_backward (dq, dk, dv, dbeta, dS0) with the fp64 oracle's
adjoint recurrence, on every supported shape family, both dtypes, both
updates, with and without S0 and dS_L, ragged tails and empty sequences;
the c3-sized workload on sampled heads; the autograd wrapper; determinism."""
import numpy as np
import pytest
import torch

import delta_rule_sequence_alpha_amd as efla
import efla_workloads as wl
import oracle
from tests._parity import TOL, dev, note, rel_err

pytestmark = pytest.mark.gpu

NAMES = ["dq", "dk", "dv", "dbeta", "dS0"]


def _case(w, seed, s0=True, dsl=True, update="exact"):
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=seed)
    if not s0:
        S0 = None
    elif S0 is None:
        S0 = torch.from_numpy(np.random.default_rng(seed + 99).standard_normal(
            (w.B, w.H, w.d_k, w.d_v)).astype(np.float32) * np.float32(0.05))
    dO, dSL = wl.output_grads(w, seed=seed, with_dS_L=dsl)
    note(f"backward {w.name} {w.dtype} B={w.B} H={w.H} L={w.L} dk={w.d_k} dv={w.d_v} "
         f"C={w.chunk} S0={s0} dSL={dsl} {update}")
    got = efla.backward(*dev(q, k, v, beta, S0, dO, dSL), chunk=w.chunk, update=update)
    torch.cuda.synchronize()
    return (q, k, v, beta, S0, dO, dSL), got


def _compare(inputs, got, tol, update="exact", sl=None):
    q, k, v, beta, S0, dO, dSL = inputs
    if sl is not None:
        q, k, v, beta, dO = q[sl], k[sl], v[sl], beta[sl], dO[sl]
        S0 = None if S0 is None else S0[sl]
        dSL = None if dSL is None else dSL[sl]
        got = [g[sl] for g in got]
    ref = oracle.backward(q, k, v, beta, S0, dO, dSL, update=update)
    errs = {n: rel_err(g, r) for n, g, r in zip(NAMES, got, ref)}
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= tol, (n, e, tol)


SHAPES = [(16, 16, 16, 33), (32, 64, 32, 100), (64, 32, 16, 50), (128, 16, 64, 70),
          (16, 128, 32, 64), (128, 128, 64, 64 * 2 + 29), (64, 128, 64, 64)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,chunk,L", SHAPES)
def test_backward_shapes(dtype, dk, dv, chunk, L):
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(name="bwd", B=2, H=2, L=L, d_k=dk, d_v=dv,
                                                  chunk=chunk, dtype=dtype)
    inputs, got = _case(w, seed=dk + dv + L)
    _compare(inputs, got, TOL[dtype])


@pytest.mark.parametrize("s0,dsl", [(False, False), (False, True), (True, False)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_optional_states(dtype, s0, dsl):
    w = wl.FORWARD_WORKLOADS["lm340m-bf16"].with_(name="bwd", B=1, H=3, L=150, dtype=dtype)
    inputs, got = _case(w, seed=5, s0=s0, dsl=dsl)
    _compare(inputs, got, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_euler(dtype):
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(name="bwd", B=2, H=2, L=64 * 3 + 5, dtype=dtype)
    inputs, got = _case(w, seed=8, update="euler")
    _compare(inputs, got, TOL[dtype], update="euler")
    # a different operator's gradient than the exact flow's
    ref_x = oracle.backward(*inputs, update="exact")
    if dtype == "f32":
        assert rel_err(got[3], ref_x[3]) > 10 * TOL[dtype]


def test_backward_stiff_f32():
    # beta up to 5 and keys with lambda up to 1e4: alpha = 1/lambda, d alpha/d beta ~ 0
    w = wl.FORWARD_WORKLOADS["long-stiff-f32"].with_(name="bwd", B=1, H=2, L=64 * 4 + 9)
    inputs, got = _case(w, seed=2, s0=False)
    _compare(inputs, got, TOL["f32"])


def test_backward_tiny_f32():
    w = wl.FORWARD_WORKLOADS["tiny-f32"]
    inputs, got = _case(w, seed=0, s0=False)
    _compare(inputs, got, TOL["f32"])


def test_backward_full_size_sampled_heads():
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"]
    inputs, got = _case(w, seed=0)
    for b, h in [(0, 0), (3, 15)]:
        _compare(inputs, got, TOL["bf16"], sl=(slice(b, b + 1), slice(h, h + 1)))


def test_backward_deterministic():
    w = wl.FORWARD_WORKLOADS["lm340m-bf16"].with_(name="bwd", B=2, H=2, L=300)
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=3)
    dO, dSL = wl.output_grads(w, seed=3)
    note("backward determinism")
    args = dev(q, k, v, beta, S0, dO, dSL)
    a = efla.backward(*args, chunk=w.chunk)
    b = efla.backward(*args, chunk=w.chunk)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_empty_and_single_token():
    w = wl.FORWARD_WORKLOADS["tiny-f32"].with_(name="bwd", B=1, H=2, L=0)
    q, k, v, beta, _ = wl.forward_inputs(w, seed=1)
    dO, dSL = wl.output_grads(w, seed=1)
    note("backward L=0")
    dq, dk, dv, dbeta, dS0 = efla.backward(*dev(q, k, v, beta, None, dO, dSL), chunk=16)
    torch.cuda.synchronize()
    assert torch.equal(dS0.cpu(), dSL)
    w1 = w.with_(L=1)
    inputs, got = _case(w1, seed=4)
    _compare(inputs, got, TOL["f32"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_autograd_function(dtype):
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(name="bwd", B=1, H=2, L=100, dtype=dtype)
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=6)
    dO, dSL = wl.output_grads(w, seed=6)
    note(f"autograd function {dtype}")
    leaves = [x.cuda().requires_grad_() for x in (q, k, v, beta, S0)]
    o, S_L = efla.efla(*leaves, chunk=w.chunk)
    loss = (o.float() * dO.cuda().float()).sum() + (S_L * dSL.cuda()).sum()
    loss.backward()
    torch.cuda.synchronize()
    got = [x.grad for x in leaves]
    _compare((q, k, v, beta, S0, dO, dSL), got, TOL[dtype])


@pytest.mark.parametrize("recipe,dtype,H,L", [("long-stiff-f32", "f32", 2, 64 * 20 + 7),
                                              ("lm1.3b-bf16", "bf16", 2, 64 * 20 + 7),
                                              ("long-stiff-f32", "f32", 4, 4096)])
def test_backward_segmented_few_long_sequences(recipe, dtype, H, L):
    # few long sequences: both backward scans run split over L into segments
    # (segment maps, their composition, replay), as the forward's segmented path
    w = wl.FORWARD_WORKLOADS[recipe].with_(name="bwd-seg", B=1, H=H, L=L, dtype=dtype)
    inputs, got = _case(w, seed=9)
    _compare(inputs, got, TOL[dtype])
