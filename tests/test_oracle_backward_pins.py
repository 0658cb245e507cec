"""Pins of the oracle's backward (the adjoint recurrence) against things other
than itself: central finite differences of the oracle's forward (itself pinned
in test_oracle_pins.py), torch's automatic differentiation of an fp64
recurrence written independently here, and closed forms of the derivatives of
alpha = (1 - e^{-beta lambda}) / lambda ("Exact Flow Linear Attention: Exact
Solution from Continuous-Time Dynamics", Technical Summary, Methodology 3).

The loss is Loss = <dO, o> + <dS_L, S_L>, so its gradients with respect to the
inputs are what a training step back-propagates through the operator.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _inputs(rng, B, H, L, dk, dv, lam_scale=1.0, s0=True, dsl=True, beta_hi=1.0):
    q = rng.standard_normal((B, H, L, dk))
    g = rng.standard_normal((B, H, L, dk))
    k = g / np.linalg.norm(g, axis=-1, keepdims=True) * np.sqrt(
        lam_scale * rng.uniform(0.2, 2.0, (B, H, L, 1)))
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0.05, beta_hi, (B, H, L))
    S0 = 0.3 * rng.standard_normal((B, H, dk, dv)) if s0 else None
    dO = rng.standard_normal((B, H, L, dv))
    dSL = rng.standard_normal((B, H, dk, dv)) if dsl else None
    return q, k, v, beta, S0, dO, dSL


def _loss(q, k, v, beta, S0, dO, dSL, update):
    o, SL = oracle.forward(q, k, v, beta, S0, update=update)
    val = float(np.sum(dO * o))
    if dSL is not None:
        val += float(np.sum(dSL * SL))
    return val


def _torch_grads(q, k, v, beta, S0, dO, dSL, update):
    """Autograd through a plain fp64 token loop (written here, not the oracle's)."""
    t = {n: torch.tensor(x, dtype=torch.float64, requires_grad=True)
         for n, x in dict(q=q, k=k, v=v, beta=beta).items()}
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    S0t = torch.tensor(S0 if S0 is not None else np.zeros((B, H, dk, dv)),
                       dtype=torch.float64, requires_grad=True)
    S = S0t
    outs = []
    for i in range(L):
        kt, vt, qt, bt = t["k"][:, :, i], t["v"][:, :, i], t["q"][:, :, i], t["beta"][:, :, i]
        lam = (kt * kt).sum(-1)
        a = bt if update == "euler" else -torch.expm1(-bt * lam) / lam
        # S <- exp(-beta k k^T) S + (integral of the input): (I - a k k^T) S + a k v^T
        Ak = torch.eye(dk, dtype=torch.float64) - a[..., None, None] * kt[..., :, None] * kt[..., None, :]
        S = Ak @ S + a[..., None, None] * kt[..., :, None] * vt[..., None, :]
        outs.append((S * qt[..., :, None]).sum(-2))
    o = torch.stack(outs, 2)
    loss = (o * torch.tensor(dO)).sum()
    if dSL is not None:
        loss = loss + (S * torch.tensor(dSL)).sum()
    loss.backward()
    return (t["q"].grad.numpy(), t["k"].grad.numpy(), t["v"].grad.numpy(),
            t["beta"].grad.numpy(), S0t.grad.numpy())


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("update", ["exact", "euler"])
@pytest.mark.parametrize("B,H,L,dk,dv,s0,dsl", [(1, 1, 5, 3, 2, True, True),
                                               (2, 1, 9, 4, 3, False, True),
                                               (1, 2, 7, 2, 5, True, False)])
def test_backward_matches_finite_differences_elementwise(update, B, H, L, dk, dv, s0, dsl):
    rng = np.random.default_rng(zlib.crc32(repr((B, H, L, dk, dv, update)).encode()))
    q, k, v, beta, S0, dO, dSL = _inputs(rng, B, H, L, dk, dv, s0=s0, dsl=dsl)
    grads = oracle.backward(q, k, v, beta, S0, dO, dSL, update=update)
    names = ["q", "k", "v", "beta", "S0"]
    args = dict(q=q, k=k, v=v, beta=beta, S0=S0 if S0 is not None else np.zeros((B, H, dk, dv)))
    h = 1e-6
    for name, g in zip(names, grads):
        x = args[name]
        fd = np.empty_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap = dict(args, **{name: xp})
            am = dict(args, **{name: xm})
            fd[idx] = (_loss(ap["q"], ap["k"], ap["v"], ap["beta"], ap["S0"], dO, dSL, update) -
                       _loss(am["q"], am["k"], am["v"], am["beta"], am["S0"], dO, dSL, update)) / (2 * h)
        assert _rel(g, fd) < 1e-7, (name, _rel(g, fd))


@pytest.mark.parametrize("update", ["exact", "euler"])
@pytest.mark.parametrize("L,dk,dv,s0,dsl,lam_scale", [(70, 6, 5, True, True, 1.0),
                                                      (130, 4, 4, False, False, 1.0),
                                                      (66, 5, 3, True, True, 30.0),
                                                      (1, 3, 3, True, True, 1.0)])
def test_backward_matches_autograd(update, L, dk, dv, s0, dsl, lam_scale):
    # L past 64 and 128 crosses the oracle's state copies; lam_scale = 30 with
    # beta up to 1 puts beta lambda deep in the stiff range (exact update only:
    # the Euler step is unstable there, and its gradients grow without bound)
    if update == "euler" and lam_scale > 1:
        pytest.skip("explicit Euler diverges for beta lambda > 2")
    rng = np.random.default_rng(L * 100 + dk)
    q, k, v, beta, S0, dO, dSL = _inputs(rng, 2, 2, L, dk, dv, lam_scale=lam_scale, s0=s0, dsl=dsl)
    got = oracle.backward(q, k, v, beta, S0, dO, dSL, update=update)
    ref = _torch_grads(q, k, v, beta, S0, dO, dSL, update)
    for name, a, b in zip(["dq", "dk", "dv", "dbeta", "dS0"], got, ref):
        assert _rel(a, b) < 1e-11, (name, _rel(a, b))


def test_alpha_derivatives_closed_forms_and_limits():
    beta = np.array([0.0, 0.3, 1.0, 2.0, 0.7, 5.0, 1e-8, 1.0, 3.0])
    lam = np.array([1.0, 0.0, 1e-12, 0.2, 0.6, 40.0, 1.0, 1e4, 0.18])
    db, dl = oracle.alpha_grad(beta, lam)
    x = beta * lam
    # d alpha / d beta = e^{-beta lambda} exactly (derivative of 1 - e^{-x} over lambda)
    np.testing.assert_allclose(db, np.exp(-x), rtol=1e-15, atol=0)
    # lambda -> 0: alpha -> beta - beta^2 lambda / 2 + ..., so d alpha / d lambda -> -beta^2 / 2
    assert dl[1] == -0.3 ** 2 / 2
    # stiff end: alpha -> 1 / lambda, derivative -> -1 / lambda^2
    assert abs(dl[7] / (-1.0 / 1e8) - 1) < 1e-12
    # central differences of the oracle's alpha everywhere the formula is smooth
    for b, l, gb, gl in zip(beta, lam, db, dl):
        hb = 1e-6 * max(1.0, b)
        fd_b = (oracle.alpha_scalar(b + hb, l) - oracle.alpha_scalar(b - hb, l)) / (2 * hb)
        assert abs(fd_b - gb) <= 1e-8 * max(1.0, abs(gb))
        if l > 1e-3:
            hl = 1e-6 * l
            fd_l = (oracle.alpha_scalar(b, l + hl) - oracle.alpha_scalar(b, l - hl)) / (2 * hl)
            assert abs(fd_l - gl) <= 1e-7 * max(1e-12, abs(gl)) + 1e-14
    # both branches of d alpha / d lambda meet at |x| = 1/2 (series vs closed form)
    for xb in (0.5 - 1e-12, 0.5 + 1e-12):
        _, a_lo = oracle.alpha_grad(np.array([1.0]), np.array([xb]))
        g_ref = (1 - (1 + xb) * np.exp(-xb)) / xb ** 2
        assert abs(-a_lo[0] - g_ref) < 1e-13
    # Euler: alpha = beta
    db_e, dl_e = oracle.alpha_grad(beta, lam, update="euler")
    assert np.all(db_e == 1.0) and np.all(dl_e == 0.0)


def test_backward_zero_key_token_and_stiff_limit():
    rng = np.random.default_rng(7)
    q, k, v, beta, S0, dO, dSL = _inputs(rng, 1, 1, 6, 4, 3)
    k[0, 0, 2] = 0.0                  # lambda = 0: alpha = beta, update is the identity
    k[0, 0, 4] *= 30.0                # beta lambda >> 50: alpha = 1 / lambda to rounding
    beta[0, 0, 4] = 2.0
    dq, dk, dv, dbeta, dS0 = oracle.backward(q, k, v, beta, S0, dO, dSL)
    # the identity update leaves v_2 and beta_2 without influence
    assert np.all(dv[0, 0, 2] == 0.0) and dbeta[0, 0, 2] == 0.0
    # d alpha / d beta = e^{-beta lambda} underflows in the stiff token
    assert abs(dbeta[0, 0, 4]) < 1e-20
    # a zero key still receives a gradient (the update's first-order term in k)
    h = 1e-6
    for i in range(4):
        kp, km = k.copy(), k.copy()
        kp[0, 0, 2, i] += h
        km[0, 0, 2, i] -= h
        fd = (_loss(q, kp, v, beta, S0, dO, dSL, "exact") -
              _loss(q, km, v, beta, S0, dO, dSL, "exact")) / (2 * h)
        assert abs(fd - dk[0, 0, 2, i]) < 1e-7 * max(1.0, abs(fd))


def test_backward_empty_sequence():
    rng = np.random.default_rng(3)
    q, k, v, beta, S0, dO, dSL = _inputs(rng, 1, 2, 0, 3, 2)
    dq, dk, dv, dbeta, dS0 = oracle.backward(q, k, v, beta, S0, dO, dSL)
    assert dq.shape == (1, 2, 0, 3) and dbeta.shape == (1, 2, 0)
    np.testing.assert_array_equal(dS0, dSL)   # S_L = S0 when there are no tokens
