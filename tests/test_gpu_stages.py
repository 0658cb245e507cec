"""Parity of each stage of the staged chunked path against the fp64 oracle.

Stage 1 (coefficients), stage 2 (UT transform: W, U and A = tril(Q K^T) per
chunk) and stage 3 (state scan fed with the oracle's own W, U, A) are each
compared element by element with the oracle on the same seeded inputs.
"""
import numpy as np
import pytest
import torch

import delta_rule_sequence_alpha_amd as efla
import efla_workloads as wl
import oracle
from tests._parity import TOL, dev, note, rel_err

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _inputs(dtype, B, H, L, dk, dv, seed, recipe="stiff"):
    base = {"stiff": "long-stiff-f32", "lm1.3b": "lm1.3b-bf16", "tiny": "tiny-f32"}[recipe]
    w = wl.FORWARD_WORKLOADS[base].with_(B=B, H=H, L=L, d_k=dk, d_v=dv, dtype=dtype)
    return wl.forward_inputs(w, seed=seed)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk", [16, 32, 64, 128])
def test_coefficients(dtype, dk):
    note(f"coefficients {dtype} dk={dk}")
    q, k, v, beta, _ = _inputs(dtype, 2, 3, 257, dk, 16, seed=dk)
    # edge tokens: k = 0 (lambda = 0), beta = 0, and a very stiff token
    k[0, 0, 0] = 0
    beta[0, 0, 1] = 0
    k[0, 1, 2] *= 30
    beta[0, 1, 2] = 5.0
    alpha_g, lam_g = efla.coefficients(dev(k), dev(beta))
    torch.cuda.synchronize()
    alpha_r, lam_r = oracle.coefficients(k, beta)
    a = alpha_g.cpu().double().numpy()
    lmb = lam_g.cpu().double().numpy()
    assert a[0, 0, 0] == pytest.approx(float(beta[0, 0, 0]), rel=1e-7)
    assert a[0, 0, 1] == 0.0
    nz = alpha_r > 0
    rel = lambda x, r: float(np.max(np.abs(x - r) / np.maximum(np.abs(r), 1e-30)))  # noqa: E731
    # lambda = |k|^2 accumulated in fp32: d_k non-negative terms, each product
    # rounded at most once, so the relative error is at most (d_k + 1) 2^-24
    lam_tol = (dk + 1) * 2.0 ** -24
    e_lam = rel(lmb, lam_r)
    # alpha as a function of (beta, lambda): against the oracle's alpha at the
    # GPU's own lambda, 1e-6 relative (series, exp2 and reciprocal in fp32
    # against expm1 in fp64)
    alpha_at_g = oracle.alpha(beta.double().numpy(), lmb)
    e_fun = rel(a[nz], alpha_at_g[nz])
    # end to end: |d ln(alpha) / d ln(lambda)| = |x / (e^x - 1) - 1| <= 1
    # (x = beta lambda), so lambda's error reaches alpha at most once
    e_all = rel(a[nz], alpha_r[nz])
    print(f"  lambda {e_lam:.2e} (<= {lam_tol:.2e})  alpha(beta, lambda) {e_fun:.2e}  "
          f"alpha {e_all:.2e}", flush=True)
    assert e_lam <= lam_tol
    assert e_fun <= 1e-6
    assert e_all <= 1e-6 + lam_tol


def _ref_aqk(q, k, chunk):
    q = q.double().numpy()
    k = k.double().numpy()
    B, H, L, _ = k.shape
    n = (L + chunk - 1) // chunk
    A = np.zeros((B, H, n, chunk, chunk))
    for c in range(n):
        s, e = c * chunk, min(L, (c + 1) * chunk)
        A[:, :, c, :e - s, :e - s] = np.tril(q[:, :, s:e] @ np.swapaxes(k[:, :, s:e], -1, -2))
    return A


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,chunk,L", [(16, 16, 16, 64), (32, 64, 32, 100), (128, 128, 64, 200),
                                           (64, 128, 64, 64), (128, 16, 16, 37), (16, 128, 64, 150)])
def test_ut_transform(dtype, dk, dv, chunk, L):
    note(f"ut_transform {dtype} dk={dk} dv={dv} C={chunk} L={L}")
    q, k, v, beta, _ = _inputs(dtype, 1, 2, L, dk, dv, seed=L + dk)
    alpha_r, _ = oracle.coefficients(k, beta)
    alpha32 = torch.from_numpy(alpha_r.astype(np.float32))
    W, U, A = efla.ut_transform(*dev(q, k, v, alpha32), chunk=chunk)
    torch.cuda.synchronize()
    _, Wr, Ur = oracle.ut_transform(k, v, alpha32.double().numpy(), chunk)
    tol = TOL[dtype]
    assert rel_err(W, Wr) <= tol
    assert rel_err(U, Ur) <= tol
    assert rel_err(A, _ref_aqk(q, k, chunk)) <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,chunk,L,with_s0", [(16, 16, 16, 64, False), (128, 128, 64, 300, True),
                                                   (64, 32, 32, 77, True), (32, 128, 64, 130, False)])
def test_chunk_scan_on_oracle_intermediates(dtype, dk, dv, chunk, L, with_s0):
    note(f"chunk_scan {dtype} dk={dk} dv={dv} C={chunk} L={L} S0={with_s0}")
    q, k, v, beta, _ = _inputs(dtype, 2, 2, L, dk, dv, seed=L * 3 + dv)
    S0 = (torch.randn(2, 2, dk, dv, generator=torch.Generator().manual_seed(5)) * 0.1) if with_s0 else None
    alpha_r, _ = oracle.coefficients(k, beta)
    _, Wr, Ur = oracle.ut_transform(k, v, alpha_r, chunk)
    Ar = _ref_aqk(q, k, chunk)
    cast = lambda x: torch.from_numpy(x).to(DT[dtype])  # noqa: E731
    o, S_L = efla.chunk_scan(*dev(q, k, cast(Wr), cast(Ur), cast(Ar), S0), chunk=chunk)
    torch.cuda.synchronize()
    o_r, S_r = oracle.forward(q, k, v, beta, S0)
    assert rel_err(o, o_r) <= TOL[dtype]
    assert rel_err(S_L, S_r) <= TOL[dtype]
