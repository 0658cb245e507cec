"""Parity of the Euler (delta rule) variant, update="euler" (alpha := beta),
with the fp64 oracle's Euler recurrence, on every path that takes it: the
fused and staged forward, the decode step and the coefficient stage.

Inputs follow the lm1.3b recipe (lambda ~ 1, beta < 1), where the explicit
Euler step is stable.  In the stiff regime it is not (see the oracle pins):
the last test shows the GPU kernels' Euler state diverging there while the
exact flow's stays bounded and equal to the oracle's."""
import pytest
import torch

import delta_rule_sequence_alpha_amd as efla
import efla_workloads as wl
import oracle
from tests._parity import TOL, dev, note, rel_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("path,dtype", [("fused", "bf16"), ("staged", "bf16"), ("staged", "f32")])
@pytest.mark.parametrize("dk,dv,chunk,L", [(128, 128, 64, 64 * 3 + 29), (64, 32, 32, 100),
                                           (16, 16, 16, 33)])
def test_forward_euler(path, dtype, dk, dv, chunk, L):
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(B=2, H=2, L=L, d_k=dk, d_v=dv, chunk=chunk,
                                                  dtype=dtype)
    note(f"forward euler {path} {dtype} dk={dk} dv={dv} C={chunk} L={L}")
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=11)
    o, S_L = efla.forward(*dev(q, k, v, beta, S0), chunk=chunk, path=path, update="euler")
    torch.cuda.synchronize()
    o_r, S_r = oracle.forward(q, k, v, beta, S0, update="euler")
    eo, es = rel_err(o, o_r), rel_err(S_L, S_r)
    print(f"  err o={eo:.3e} S_L={es:.3e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]
    # and it is a different operator from the exact flow on the same inputs
    o_x, _ = oracle.forward(q, k, v, beta, S0, update="exact")
    assert rel_err(o, o_x) > 10 * TOL[dtype] or dtype == "bf16"


def test_forward_euler_full_size_sampled_heads():
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"]
    note("forward euler lm1.3b-bf16 full size")
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=0)
    o, S_L = efla.forward(*dev(q, k, v, beta, S0), chunk=w.chunk, update="euler")
    torch.cuda.synchronize()
    for b, h in [(0, 0), (2, 7)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_r, S_r = oracle.forward(q[sl], k[sl], v[sl], beta[sl], S0[sl], update="euler")
        assert rel_err(o[sl], o_r) <= TOL["bf16"] and rel_err(S_L[sl], S_r) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_euler(dtype):
    w = wl.DecodeWorkload("d", 6, 4, 128, 128, 4, dtype)
    note(f"decode euler {dtype}")
    S = wl.decode_state(w, seed=3)
    Sd = dev(S)
    S_ref = S.double().numpy()
    for step in range(4):
        q, k, v, beta = wl.decode_tokens(w, step, seed=3)
        o = efla.decode_step(*dev(q, k, v, beta), Sd, update="euler")
        torch.cuda.synchronize()
        o_r, S_ref = oracle.decode(q, k, v, beta, S_ref, update="euler")
        assert rel_err(o, o_r) <= TOL[dtype]
        assert rel_err(Sd, S_ref) <= 1e-5


def test_coefficients_euler_is_beta():
    w = wl.FORWARD_WORKLOADS["long-stiff-f32"].with_(B=1, H=2, L=300)
    note("coefficients euler")
    _, k, _, beta, _ = wl.forward_inputs(w, seed=4)
    a, lam = efla.coefficients(*dev(k, beta), update="euler")
    torch.cuda.synchronize()
    assert torch.equal(a.cpu(), beta)
    _, lam_r = oracle.coefficients(k, beta)
    assert rel_err(lam, lam_r) <= 1e-6


@pytest.mark.parametrize("path", ["staged", "segmented"])
def test_stiff_recipe_euler_diverges_exact_stays_bounded(path):
    """The stiff regime the exact flow is for (Technical Summary, Problem
    Statement): with beta lambda up to ~5e4 the Euler transition
    I - beta k k^T has an eigenvalue 1 - beta lambda far below -1 along k, so
    the Euler state blows up within a few such tokens, while the exact
    transition's eigenvalue e^{-beta lambda} stays in (0, 1] and the state
    stays bounded.  Same kernels, same inputs, only alpha differs."""
    w = wl.FORWARD_WORKLOADS["long-stiff-f32"].with_(B=1, H=2, L=64 * 40)
    note(f"stiff exact vs euler {path}")
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=43)
    args = dev(q, k, v, beta, S0)
    o_x, S_x = efla.forward(*args, chunk=w.chunk, path=path)
    o_e, S_e = efla.forward(*args, chunk=w.chunk, path=path, update="euler")
    torch.cuda.synchronize()
    # exact: finite, and (each transition a contraction, ||I - alpha k k^T|| <= 1)
    # |S_L|_F at most |S0|_F plus the tokens' injections |alpha k v^T|_F =
    # alpha |k| |v| <= min(|v| / |k|, beta |k| |v|)  (alpha <= 1/lambda, alpha <= beta)
    assert torch.isfinite(o_x).all() and torch.isfinite(S_x).all()
    kn = k.double().norm(dim=-1)
    vn = v.double().norm(dim=-1)
    inj = torch.minimum(vn / kn.clamp_min(1e-300), beta.double() * kn * vn)
    bound = inj.sum(dim=-1)
    if S0 is not None:
        bound = bound + S0.double().norm(dim=(-2, -1))
    assert bool((S_x.double().cpu().norm(dim=(-2, -1)) <= bound * (1 + 1e-6)).all())
    # Euler: overflowed (non-finite) or astronomically large
    big = (~torch.isfinite(S_e)).any() or float(S_e.abs().max()) > 1e30
    print(f"  exact |S_L| {float(S_x.abs().max()):.3e}; euler non-finite "
          f"{float((~torch.isfinite(S_e)).float().mean()):.2f}", flush=True)
    assert big
    # the exact result is the oracle's
    o_r, S_r = oracle.forward(q, k, v, beta, S0)
    assert rel_err(o_x, o_r) <= TOL["f32"] and rel_err(S_x, S_r) <= TOL["f32"]
