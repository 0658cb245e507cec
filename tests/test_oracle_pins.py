"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself:
library matrix exponentials, the exact solution of the zero-order-hold ODE
(Van Loan block exponential, RK4, the scalar closed form), algebraic
invariants the pages state, and brute force on tiny inputs.  Sources are in
"Exact Flow Linear Attention: Exact Solution from Continuous-Time Dynamics"
(gist.science Technical Summary): Problem Statement (Euler reading, stiffness),
Methodology 1 (ODE), 2 (rank-1 power identity, closed-form exponential),
3 (update rule, alpha, chunkwise parallelism), Key Contributions (contraction
along k by e^{-beta lambda}).
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
from tests._numpy_recurrence import dense_forward

RNG = np.random.default_rng(12345)


def _rand_key(rng, d, lam):
    g = rng.standard_normal(d)
    return g / np.linalg.norm(g) * np.sqrt(lam)


def _one_step(k, v, beta, S, q=None):
    """Oracle decode step on a single (n, h) = (0, 0) head."""
    dk, dv = S.shape
    if q is None:
        q = np.zeros(dk)
    o, Sn = oracle.decode(q[None, None], k[None, None], v[None, None],
                          np.array([[beta]]), S[None, None])
    return o[0, 0], Sn[0, 0]


def _taylor_expm(M, terms=60):
    """exp(M) by scaling and squaring of a truncated Taylor series."""
    nrm = np.linalg.norm(M, 1)
    s = max(0, int(np.ceil(np.log2(nrm))) + 1) if nrm > 0 else 0
    X = M / (2.0 ** s)
    E = np.eye(M.shape[0])
    term = np.eye(M.shape[0])
    for n in range(1, terms):
        term = term @ X / n
        E = E + term
    for _ in range(s):
        E = E @ E
    return E


def _exact_flow(k, v, beta, S):
    """Exact solution of dS/dt = -k k^T S + k v^T over [0, beta] (Van Loan)."""
    dk, dv = S.shape
    M = np.zeros((dk + dv, dk + dv))
    M[:dk, :dk] = -np.outer(k, k)
    M[:dk, dk:] = np.outer(k, v)
    E = scipy.linalg.expm(beta * M)
    return E[:dk, :dk] @ S + E[:dk, dk:]


# --- P1: closed-form matrix exponential (Methodology 2) ---------------------

@pytest.mark.parametrize("d", [2, 3, 4, 8])
@pytest.mark.parametrize("lam", [1e-6, 1e-2, 0.7, 3.0, 40.0, 1e4])
def test_p1_closed_form_exponential(d, lam):
    rng = np.random.default_rng(d * 1000 + int(lam * 10))
    k = _rand_key(rng, d, lam)
    A = np.outer(k, k)
    for beta in [0.0, 0.013, 0.5, 1.0, 5.0]:
        a = oracle.alpha(beta, k @ k)
        assert a == pytest.approx(oracle.alpha_scalar(beta, k @ k), rel=1e-15, abs=0)
        closed = np.eye(d) - a * A
        ref = scipy.linalg.expm(-beta * A)
        # scaling and squaring loses about one ulp per squaring: log2(beta*lambda) of them
        tol = 1e-12 * (1.0 + np.log2(1.0 + beta * lam))
        assert np.max(np.abs(closed - ref)) <= tol
        if beta * lam <= 60:
            tay = _taylor_expm(-beta * A)
            assert np.max(np.abs(closed - tay)) <= 1e-12


@pytest.mark.parametrize("d", [3, 8])
def test_p1_oracle_homogeneous_step_is_expm(d):
    """With v = 0 one oracle step applies exactly e^{-beta k k^T} to S."""
    rng = np.random.default_rng(7)
    for lam, beta in [(0.3, 0.9), (2.0, 1.7), (50.0, 0.2), (1e-5, 3.0)]:
        k = _rand_key(rng, d, lam)
        S = rng.standard_normal((d, d + 2))
        _, Sn = _one_step(k, np.zeros(d + 2), beta, S)
        ref = scipy.linalg.expm(-beta * np.outer(k, k)) @ S
        assert np.max(np.abs(Sn - ref)) <= 1e-12 * max(1.0, np.max(np.abs(S)))


# --- P2: rank-1 power identity (Methodology 2) -------------------------------

@pytest.mark.parametrize("d", [2, 5, 16])
def test_p2_rank1_power_identity(d):
    rng = np.random.default_rng(d)
    k = rng.standard_normal(d)
    A = np.outer(k, k)
    lam = k @ k
    for n in range(1, 13):
        An = np.linalg.matrix_power(A, n)
        assert np.max(np.abs(An - lam ** (n - 1) * A)) <= 1e-13 * np.max(np.abs(An))


# --- P3: one oracle step is the exact ODE flow (Methodology 1-3) ------------

@pytest.mark.parametrize("dk,dv", [(1, 1), (3, 5), (8, 4), (16, 16)])
def test_p3_step_equals_exact_ode_flow(dk, dv):
    rng = np.random.default_rng(100 + dk * dv)
    for lam, beta in [(0.01, 0.5), (1.0, 1.0), (4.0, 0.3), (16.0, 1.0), (100.0, 5.0)]:
        k = _rand_key(rng, dk, lam)
        v = rng.standard_normal(dv)
        S = rng.standard_normal((dk, dv))
        _, Sn = _one_step(k, v, beta, S)
        ref = _exact_flow(k, v, beta, S)
        assert np.max(np.abs(Sn - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_p3_step_equals_rk4_integration():
    rng = np.random.default_rng(3)
    dk, dv = 6, 3
    k = _rand_key(rng, dk, 2.5)
    v = rng.standard_normal(dv)
    S0 = rng.standard_normal((dk, dv))
    beta = 0.8
    A, b = np.outer(k, k), np.outer(k, v)
    f = lambda S: -A @ S + b  # noqa: E731
    n = 10_000
    h = beta / n
    S = S0.copy()
    for _ in range(n):
        k1 = f(S)
        k2 = f(S + 0.5 * h * k1)
        k3 = f(S + 0.5 * h * k2)
        k4 = f(S + h * k3)
        S = S + h / 6.0 * (k1 + 2 * k2 + 2 * k3 + k4)
    _, Sn = _one_step(k, v, beta, S0)
    assert np.max(np.abs(Sn - S)) <= 1e-10


def test_p3_scalar_closed_form():
    """d_k = d_v = 1: dS/dt = -k^2 S + k v has S(b) = e^{-b k^2} S0 + (1 - e^{-b k^2}) v / k."""
    for k, v, beta, S0 in [(2.0, 3.0, 0.5, 1.0), (0.1, -1.0, 0.7, 0.25), (-3.0, 0.5, 2.0, -4.0)]:
        q = 1.5
        o, Sn = _one_step(np.array([k]), np.array([v]), beta, np.array([[S0]]), np.array([q]))
        ref = np.exp(-beta * k * k) * S0 + (1.0 - np.exp(-beta * k * k)) * v / k
        assert Sn[0, 0] == pytest.approx(ref, rel=1e-14, abs=1e-15)
        assert o[0] == pytest.approx(ref * q, rel=1e-14, abs=1e-15)


@pytest.mark.parametrize("dk,dv", [(4, 7), (7, 4)])
def test_p3_sequence_matches_exact_flows_and_readout(dk, dv):
    """A whole forward call equals chained exact ODE flows, read out as o_t = S_t^T q_t.

    d_k != d_v so that a transposed state or readout cannot pass.
    """
    rng = np.random.default_rng(dk * 31 + dv)
    B, H, L = 2, 2, 9
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk)) * rng.uniform(0.2, 2.0, (B, H, L, 1))
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0, 3, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, SL = oracle.forward(q, k, v, beta, S0)
    for b in range(B):
        for h in range(H):
            S = S0[b, h].copy()
            for t in range(L):
                S = _exact_flow(k[b, h, t], v[b, h, t], beta[b, h, t], S)
                np.testing.assert_allclose(o[b, h, t], S.T @ q[b, h, t], rtol=0, atol=1e-11)
            np.testing.assert_allclose(SL[b, h], S, rtol=0, atol=1e-11)


# --- P4: contraction along the key direction (Key Contributions) ------------

@pytest.mark.parametrize("lam,beta", [(0.5, 0.5), (3.0, 1.0), (20.0, 0.25), (1e4, 5.0)])
def test_p4_contraction_along_key(lam, beta):
    rng = np.random.default_rng(int(lam * 7 + beta * 3))
    dk, dv = 8, 5
    k = _rand_key(rng, dk, lam)
    v = rng.standard_normal(dv)
    S = rng.standard_normal((dk, dv))
    _, Sn = _one_step(k, v, beta, S)
    decay = np.exp(-beta * lam)
    np.testing.assert_allclose(k @ Sn, decay * (k @ S) + (1 - decay) * v,
                               rtol=0, atol=1e-13 * max(1.0, np.sqrt(lam)) * 10)
    # every direction orthogonal to k is left alone
    Q, _ = np.linalg.qr(np.column_stack([k, rng.standard_normal((dk, dk - 1))]))
    for i in range(1, dk):
        u = Q[:, i]
        np.testing.assert_allclose(u @ Sn, u @ S, rtol=0, atol=1e-13 * 10)


# --- P5: small-beta limit is the Euler (delta rule) step (Problem Statement) -

def test_p5_small_beta_limit_is_euler():
    rng = np.random.default_rng(5)
    dk, dv = 6, 6
    k = _rand_key(rng, dk, 2.0)
    v = rng.standard_normal(dv)
    S = rng.standard_normal((dk, dv))
    lam = k @ k
    diffs = []
    for beta in [1e-2, 1e-3, 1e-4]:
        a = oracle.alpha(beta, lam)
        assert abs(a - beta) <= beta * beta * lam / 2 * (1 + 1e-9)
        _, Sn = _one_step(k, v, beta, S)
        euler = S + beta * (-np.outer(k, k) @ S + np.outer(k, v))
        diffs.append(np.max(np.abs(Sn - euler)))
    # the gap shrinks like beta^2: two decades of beta -> four decades of gap
    assert 70 < diffs[0] / diffs[1] < 130
    assert 70 < diffs[1] / diffs[2] < 130


# --- P6: lambda -> 0 limit ----------------------------------------------------

def test_p6_lambda_to_zero():
    beta = 0.75
    prev = None
    for e in [-1, -3, -6, -10, -20, -100, -300]:
        lam = 10.0 ** e
        a = oracle.alpha(beta, lam)
        assert oracle.alpha_scalar(beta, lam) == pytest.approx(a, rel=1e-15)
        # alpha carries a few ulps of beta itself, which dominate once beta*lam < 1e-6
        assert abs(a - beta) <= beta * beta * lam / 2 * (1 + 1e-9) + 4 * np.finfo(float).eps * beta
        if prev is not None:
            assert abs(a - beta) <= abs(prev - beta) + 4 * np.finfo(float).eps * beta
        prev = a
    assert oracle.alpha(beta, 0.0) == beta
    assert oracle.alpha_scalar(beta, 0.0) == beta


def test_p6_zero_key_is_identity():
    rng = np.random.default_rng(6)
    S = rng.standard_normal((5, 3))
    q = rng.standard_normal(5)
    o, Sn = _one_step(np.zeros(5), rng.standard_normal(3), 0.9, S, q)
    assert np.array_equal(Sn, S)
    np.testing.assert_allclose(o, S.T @ q, rtol=1e-15, atol=0)


def test_p6_zero_beta_is_identity():
    rng = np.random.default_rng(16)
    S = rng.standard_normal((5, 3))
    _, Sn = _one_step(rng.standard_normal(5), rng.standard_normal(3), 0.0, S)
    assert np.array_equal(Sn, S)


# --- P7: stiff limit overwrites the memory along k (Problem Statement) ------

@pytest.mark.parametrize("lam,beta", [(100.0, 1.0), (1e4, 0.5), (1e4, 5.0)])
def test_p7_stiff_limit(lam, beta):
    rng = np.random.default_rng(int(lam))
    dk, dv = 8, 4
    k = _rand_key(rng, dk, lam)
    v = rng.standard_normal(dv)
    S = rng.standard_normal((dk, dv))
    assert oracle.alpha(beta, lam) * lam == pytest.approx(1.0, rel=1e-12)
    _, Sn = _one_step(k, v, beta, S)
    np.testing.assert_allclose(Sn.T @ k, v, rtol=1e-10, atol=1e-10)


# --- P8: semigroup property of the exact flow --------------------------------

def test_p8_semigroup_holds_for_exact_flow_and_fails_for_euler():
    rng = np.random.default_rng(8)
    dk, dv = 7, 5
    k = _rand_key(rng, dk, 3.0)
    v = rng.standard_normal(dv)
    S = rng.standard_normal((dk, dv))
    beta = 1.3
    _, one = _one_step(k, v, beta, S)
    _, half = _one_step(k, v, beta / 2, S)
    _, two = _one_step(k, v, beta / 2, half)
    assert np.max(np.abs(one - two)) <= 1e-14 * 10

    def euler(S, b):
        return S + b * (-np.outer(k, k) @ S + np.outer(k, v))
    assert np.max(np.abs(euler(S, beta) - euler(euler(S, beta / 2), beta / 2))) > 1e-2


# --- P9: chunk (UT) form reproduces the recurrence (Methodology 3) ----------

def _chunk_form(q, k, v, beta, S0, chunk):
    """Evaluate a sequence chunk by chunk from the oracle's T, W, U (fp64)."""
    a, _ = oracle.coefficients(k, beta)
    _, W, U = oracle.ut_transform(k, v, a, chunk)
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, L, dv))
    SL = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[b, h].copy()
            for s in range(0, L, chunk):
                e = min(L, s + chunk)
                Q, K, Wc, Uc = q[b, h, s:e], k[b, h, s:e], W[b, h, s:e], U[b, h, s:e]
                E = Uc - Wc @ S
                o[b, h, s:e] = Q @ S + np.tril(Q @ K.T) @ E
                S = S + K.T @ E
            SL[b, h] = S
    return o, SL


@pytest.mark.parametrize("chunk", [1, 2, 16, 64])
@pytest.mark.parametrize("dk,dv,L", [(16, 16, 64), (8, 12, 45), (12, 8, 100)])
def test_p9_chunk_form_equals_recurrence(chunk, dk, dv, L):
    rng = np.random.default_rng(chunk * 7 + L)
    B, H = 1, 2
    q = rng.standard_normal((B, H, L, dk))
    g = rng.standard_normal((B, H, L, dk))
    k = g / np.linalg.norm(g, axis=-1, keepdims=True) * np.exp(rng.uniform(np.log(0.1), np.log(10), (B, H, L, 1)))
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0, 5, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.1
    o, SL = oracle.forward(q, k, v, beta, S0)
    oc, SLc = _chunk_form(q, k, v, beta, S0, chunk)
    scale_o, scale_s = np.max(np.abs(o)), np.max(np.abs(SL))
    assert np.max(np.abs(oc - o)) <= 1e-12 * scale_o
    assert np.max(np.abs(SLc - SL)) <= 1e-12 * scale_s


def test_p9_ut_transform_definition_properties():
    """T is lower triangular with diag(T) = alpha; (I + G) T = diag(alpha)."""
    rng = np.random.default_rng(9)
    k = rng.standard_normal((1, 1, 40, 6))
    v = rng.standard_normal((1, 1, 40, 3))
    beta = rng.uniform(0, 2, (1, 1, 40))
    a, lam = oracle.coefficients(k, beta)
    T, W, U = oracle.ut_transform(k, v, a, 16)
    for c in range(3):
        n = min(16, 40 - 16 * c)
        Tc = T[0, 0, c, :n, :n]
        assert np.allclose(np.triu(Tc, 1), 0.0)
        np.testing.assert_allclose(np.diag(Tc), a[0, 0, 16 * c:16 * c + n], rtol=1e-15)
        K = k[0, 0, 16 * c:16 * c + n]
        G = np.tril(a[0, 0, 16 * c:16 * c + n, None] * (K @ K.T), -1)
        np.testing.assert_allclose((np.eye(n) + G) @ Tc, np.diag(a[0, 0, 16 * c:16 * c + n]), atol=1e-13)


# --- P10: norm bounds (Appendix-style stability facts, beta >= 0) -----------

def test_p10_norm_bounds():
    rng = np.random.default_rng(10)
    C, d = 32, 16
    for trial in range(5):
        g = rng.standard_normal((C, d))
        K = g / np.linalg.norm(g, axis=1, keepdims=True) * np.exp(rng.uniform(np.log(0.1), np.log(10), (C, 1)))
        beta = rng.uniform(0, 5, C)
        a, _ = oracle.coefficients(K, beta)
        T, W, _ = oracle.ut_transform(K[None], np.zeros((1, C, 1)), a[None], C)
        P = np.eye(d) - K.T @ W[0]
        assert np.linalg.norm(P, 2) <= 1 + 1e-10
        assert np.linalg.norm(T[0, 0], 2) <= beta.max() * (1 + 1e-10)
        for t in range(C):
            assert np.linalg.norm(np.eye(d) - a[t] * np.outer(K[t], K[t]), 2) <= 1 + 1e-12


# --- P11: brute force against a dense evaluation ------------------------------

@pytest.mark.parametrize("dk,dv", [(3, 3), (5, 2), (2, 6)])
def test_p11_dense_recurrence(dk, dv):
    rng = np.random.default_rng(dk * 11 + dv)
    B, H, L = 2, 3, 17
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0, 2, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, SL = oracle.forward(q, k, v, beta, S0)
    od, SLd = dense_forward(q, k, v, beta, S0)
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-13)
    np.testing.assert_allclose(SL, SLd, rtol=0, atol=1e-13)
    o0, SL0 = oracle.forward(q, k, v, beta, None)
    od0, SLd0 = dense_forward(q, k, v, beta, None)
    np.testing.assert_allclose(o0, od0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(SL0, SLd0, rtol=0, atol=1e-13)


# --- P12: the outputs are linear in (S0, V) jointly ------------------------

def test_p12_affinity():
    rng = np.random.default_rng(12)
    B, H, L, dk, dv = 1, 2, 30, 6, 4
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0, 2, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, SL = oracle.forward(q, k, v, beta, S0)
    o1, SL1 = oracle.forward(q, k, v, beta, None)
    o2, SL2 = oracle.forward(q, k, np.zeros_like(v), beta, S0)
    np.testing.assert_allclose(o, o1 + o2, atol=1e-13)
    np.testing.assert_allclose(SL, SL1 + SL2, atol=1e-13)
    o3, SL3 = oracle.forward(q, k, 2.5 * v, beta, 2.5 * S0)
    np.testing.assert_allclose(o3, 2.5 * o, atol=1e-12)
    np.testing.assert_allclose(SL3, 2.5 * SL, atol=1e-12)


# --- P13: d_v columns evolve independently ---------------------------------

def test_p13_column_permutation():
    rng = np.random.default_rng(13)
    B, H, L, dk, dv = 1, 1, 25, 5, 7
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0, 2, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv))
    perm = rng.permutation(dv)
    o, SL = oracle.forward(q, k, v, beta, S0)
    op, SLp = oracle.forward(q, k, v[..., perm], beta, S0[..., perm])
    assert np.array_equal(op, o[..., perm])
    assert np.array_equal(SLp, SL[..., perm])


# --- P14: decode steps and split/resume reproduce the whole forward -------

def test_p14_decode_steps_equal_forward():
    rng = np.random.default_rng(14)
    B, H, L, dk, dv = 2, 3, 12, 6, 5
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0, 2, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, SL = oracle.forward(q, k, v, beta, S0)
    S = S0.copy()
    for t in range(L):
        ot, S = oracle.decode(q[:, :, t], k[:, :, t], v[:, :, t], beta[:, :, t], S)
        np.testing.assert_allclose(ot, o[:, :, t], rtol=0, atol=1e-13)
    np.testing.assert_allclose(S, SL, rtol=0, atol=1e-13)


@pytest.mark.parametrize("t0", [1, 16, 23])
def test_p14_split_and_resume(t0):
    rng = np.random.default_rng(t0)
    B, H, L, dk, dv = 1, 2, 40, 6, 5
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0, 2, (B, H, L))
    o, SL = oracle.forward(q, k, v, beta)
    oa, Sa = oracle.forward(q[:, :, :t0], k[:, :, :t0], v[:, :, :t0], beta[:, :, :t0])
    ob, Sb = oracle.forward(q[:, :, t0:], k[:, :, t0:], v[:, :, t0:], beta[:, :, t0:], Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=2), o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Sb, SL, rtol=0, atol=1e-13)


# --- PE: the Euler (delta rule) variant, update="euler" (Problem Statement) -

def _dense_euler(q, k, v, beta, S0):
    """Explicit Euler step of dS/dt = -k k^T S + k v^T over [0, beta], with
    dense matrices, token by token; readout after the update."""
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, L, dv))
    SL = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.array(S0[b, h], dtype=np.float64)
            for t in range(L):
                kt, bt = k[b, h, t], beta[b, h, t]
                S = S + bt * (-np.outer(kt, kt) @ S + np.outer(kt, v[b, h, t]))
                o[b, h, t] = S.T @ q[b, h, t]
            SL[b, h] = S
    return o, SL


@pytest.mark.parametrize("dk,dv", [(4, 4), (8, 3)])
def test_pe_euler_is_the_explicit_euler_step(dk, dv):
    rng = np.random.default_rng(100 + dk)
    B, H, L = 2, 2, 13
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk)) * 0.5
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0, 1, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, SL = oracle.forward(q, k, v, beta, S0, update="euler")
    od, SLd = _dense_euler(q, k, v, beta, S0)
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(SL, SLd, rtol=0, atol=1e-12)
    # one decode step is the same update
    od1, Sd1 = oracle.decode(q[:, :, 0], k[:, :, 0], v[:, :, 0], beta[:, :, 0], S0, update="euler")
    o1, S1 = oracle.forward(q[:, :, :1], k[:, :, :1], v[:, :, :1], beta[:, :, :1], S0, update="euler")
    np.testing.assert_allclose(od1, o1[:, :, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(Sd1, S1, rtol=0, atol=1e-14)


def test_pe_euler_and_exact_agree_to_second_order_in_beta():
    """Over a whole sequence the two updates differ by O(beta^2) per token."""
    rng = np.random.default_rng(101)
    B, H, L, dk, dv = 1, 2, 9, 5, 4
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    v = rng.standard_normal((B, H, L, dv))
    base = rng.uniform(0.5, 1.0, (B, H, L))
    gaps = []
    for scale in (1e-2, 1e-3):
        oe, _ = oracle.forward(q, k, v, base * scale, None, update="exact")
        ou, _ = oracle.forward(q, k, v, base * scale, None, update="euler")
        gaps.append(np.max(np.abs(oe - ou)))
    assert 70 < gaps[0] / gaps[1] < 130


@pytest.mark.parametrize("beta_lam", [0.5, 3.0, 40.0])
def test_pe_euler_is_unstable_where_the_exact_flow_contracts(beta_lam):
    """Along k the Euler update multiplies the distance k^T S - v^T to its
    fixed point by 1 - beta lambda (below -1 once beta lambda > 2: it grows)
    where the exact flow multiplies it by e^{-beta lambda} (Key
    Contributions: contraction along the key direction)."""
    rng = np.random.default_rng(102)
    dk, dv = 6, 3
    k = _rand_key(rng, dk, 1.5)
    lam = float(k @ k)
    beta = beta_lam / lam
    v = rng.standard_normal(dv)
    S = rng.standard_normal((dk, dv))
    L = 6
    kk = np.broadcast_to(k, (1, 1, L, dk)).copy()
    vv = np.broadcast_to(v, (1, 1, L, dv)).copy()
    bb = np.full((1, 1, L), beta)
    qq = np.zeros((1, 1, L, dk))
    for update, factor in (("euler", 1.0 - beta_lam), ("exact", np.exp(-beta_lam))):
        _, SL = oracle.forward(qq, kk, vv, bb, S[None, None], update=update)
        # k^T S_t - v^T = factor^L (k^T S_0 - v^T)  (fixed point k^T S = v^T)
        got = k @ SL[0, 0] - v
        want = factor ** L * (k @ S - v)
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
    if beta_lam > 2:
        assert abs(1.0 - beta_lam) ** L > 1.0 > np.exp(-beta_lam)


# --- oracle mechanics ---------------------------------------------------------

def test_thread_count_invariance():
    rng = np.random.default_rng(15)
    B, H, L, dk, dv = 2, 4, 33, 8, 8
    args = (rng.standard_normal((B, H, L, dk)), rng.standard_normal((B, H, L, dk)),
            rng.standard_normal((B, H, L, dv)), rng.uniform(0, 2, (B, H, L)))
    o1, S1 = oracle.forward(*args, threads=1)
    o8, S8 = oracle.forward(*args, threads=8)
    assert np.array_equal(o1, o8) and np.array_equal(S1, S8)


def test_empty_sequence():
    rng = np.random.default_rng(17)
    S0 = rng.standard_normal((1, 2, 4, 3))
    o, SL = oracle.forward(np.zeros((1, 2, 0, 4)), np.zeros((1, 2, 0, 4)), np.zeros((1, 2, 0, 3)),
                           np.zeros((1, 2, 0)), S0)
    assert o.shape == (1, 2, 0, 3)
    assert np.array_equal(SL, S0)
