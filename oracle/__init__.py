"""fp64 CPU oracle for the EFLA forward operator and decode step.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product library, which must fail
loudly rather than fall back to anything here.  Nothing in this package
imports the HIP library or shares code with it.

Sources ("Exact Flow Linear Attention: Exact Solution from Continuous-Time
Dynamics", gist.science Technical Summary):
  * Methodology 2: e^{-beta A} = I - ((1 - e^{-beta lambda}) / lambda) A for the
    rank-1 A = k k^T, lambda = |k|^2.
  * Methodology 3: S_t = (I - alpha_t k_t k_t^T) S_{t-1} + alpha_t k_t v_t^T,
    alpha_t = (1 - e^{-beta_t lambda_t}) / lambda_t.
  * Readout o_t = S_t^T q_t (post-update state) and the lambda -> 0 limit
    alpha = beta are the readings stated with the operator's problem statement;
    the pages do not print the readout.
  * update="euler": the explicit Euler step of the same ODE over the interval
    beta (alpha := beta), the delta rule the pages compare against (Problem
    Statement).

Entry points
  alpha(beta, lam)           per-token coefficient (numpy, fp64)
  coefficients(k, beta)      (alpha, lambda) per token, fp64
  ut_transform(k, v, alpha, chunk)
                             per-chunk T, W = T K, U = T V by their definition
                             (a library triangular solve; see the function)
  forward(q, k, v, beta, S0, update="exact")
                             whole-sequence recurrence (C, fp64, OpenMP)
  decode(q, k, v, beta, S, update="exact")
                             one single-token step (C, fp64, OpenMP)
  alpha_grad(beta, lam, update="exact")
                             (d alpha/d beta, d alpha/d lambda) per token (C, fp64)
  backward(q, k, v, beta, S0, dO, dS_L=None, update="exact")
                             gradients (dq, dk, dv, dbeta, dS0) of a loss with
                             dLoss/do = dO and dLoss/dS_L = dS_L: the adjoint of
                             the token recurrence, backwards in time (C, fp64)

``backward`` and ``alpha_grad`` are pinned by tests/test_oracle_backward_pins.py
against central finite differences of ``forward`` and against torch's automatic
differentiation of an independently written fp64 recurrence.

Parity of ``forward``/``decode``/``alpha`` is pinned by tests/test_oracle_pins.py
against matrix exponentials, the exact ODE flow and invariants.  The chunk
quantities of ``ut_transform`` are pinned by reproducing the recurrence from
them (tests/test_oracle_pins.py, chunk-form tests).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_DP = ctypes.POINTER(ctypes.c_double)


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.efla_oracle_alpha.restype = ctypes.c_double
        lib.efla_oracle_alpha.argtypes = [ctypes.c_double, ctypes.c_double]
        lib.efla_oracle_forward.restype = ctypes.c_int
        lib.efla_oracle_forward.argtypes = [_DP] * 7 + [ctypes.c_long] * 5 + [ctypes.c_int] * 2
        lib.efla_oracle_decode.restype = ctypes.c_int
        lib.efla_oracle_decode.argtypes = [_DP] * 6 + [ctypes.c_long] * 4 + [ctypes.c_int] * 2
        lib.efla_oracle_alpha_grad.restype = None
        lib.efla_oracle_alpha_grad.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_int,
                                               _DP, _DP]
        lib.efla_oracle_backward.restype = ctypes.c_int
        lib.efla_oracle_backward.argtypes = [_DP] * 12 + [ctypes.c_long] * 5 + [ctypes.c_int] * 2
        lib.efla_oracle_max_threads.restype = ctypes.c_int
        lib.efla_oracle_max_threads.argtypes = []
        _LIB = lib
    return _LIB


def _f64(x) -> np.ndarray:
    """Exact upcast to a contiguous fp64 numpy array (bf16 and fp32 embed in fp64)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_DP)


def max_threads() -> int:
    return int(_lib().efla_oracle_max_threads())


def alpha_scalar(beta: float, lam: float) -> float:
    """The C oracle's own alpha (scalar)."""
    return float(_lib().efla_oracle_alpha(float(beta), float(lam)))


def alpha(beta, lam) -> np.ndarray:
    """alpha = (1 - e^{-beta lambda}) / lambda, and beta where lambda == 0 (fp64)."""
    beta = _f64(beta)
    lam = _f64(lam)
    beta, lam = np.broadcast_arrays(beta, lam)
    out = beta.copy()
    nz = lam != 0.0
    out[nz] = -np.expm1(-beta[nz] * lam[nz]) / lam[nz]
    return out


def coefficients(k, beta):
    """Per-token (alpha, lambda): lambda = |k|^2 over the last axis of k."""
    k = _f64(k)
    lam = np.einsum("...i,...i->...", k, k)
    return alpha(beta, lam), lam


def ut_transform(k, v, alph, chunk: int):
    """Chunk quantities of the WY/UT form, straight from their definition.

    For each chunk of ``chunk`` consecutive tokens (the last chunk may be
    shorter) with keys K [c, dk], values V [c, dv] and coefficients a [c]:
        G = strictly_lower(diag(a) K K^T)
        T = (I + G)^{-1} diag(a)          (solved, not inverted, in fp64)
        W = T K,  U = T V
    Returns (T, W, U) with W, U laid out like k, v ([..., L, d]) and T as
    [..., n_chunks, chunk, chunk] (zero-padded for a short last chunk).
    The WY/UT scheme is only named on the pages (Methodology 3); these
    definitions are the reading that makes a chunk reproduce the recurrence,
    which the pin tests check.
    """
    from scipy.linalg import solve_triangular

    k = _f64(k)
    v = _f64(v)
    alph = _f64(alph)
    L = k.shape[-2]
    lead = k.shape[:-2]
    nchunks = (L + chunk - 1) // chunk
    W = np.zeros_like(k)
    U = np.zeros_like(v)
    T = np.zeros(lead + (nchunks, chunk, chunk))
    for idx in np.ndindex(*lead):
        for c in range(nchunks):
            s, e = c * chunk, min(L, (c + 1) * chunk)
            K = k[idx][s:e]
            V = v[idx][s:e]
            a = alph[idx][s:e]
            G = np.tril(a[:, None] * (K @ K.T), -1)
            Tc = solve_triangular(np.eye(e - s) + G, np.diag(a), lower=True, unit_diagonal=True)
            T[idx + (c, slice(0, e - s), slice(0, e - s))] = Tc
            W[idx][s:e] = Tc @ K
            U[idx][s:e] = Tc @ V
    return T, W, U


def _euler(update: str) -> int:
    if update not in ("exact", "euler"):
        raise ValueError(f"unknown update {update!r}")
    return int(update == "euler")


def forward(q, k, v, beta, S0=None, threads: int = 0, update: str = "exact"):
    """Token-by-token recurrence in fp64.  Returns (o [B,H,L,dv], S_L [B,H,dk,dv]).

    q, k: [B,H,L,dk]; v: [B,H,L,dv]; beta: [B,H,L]; S0: [B,H,dk,dv] or None.
    update: "exact" (alpha from the exact flow) or "euler" (alpha = beta).
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    if q.shape != (B, H, L, dk) or v.shape != (B, H, L, dv) or beta.shape != (B, H, L):
        raise ValueError("shape mismatch")
    s0 = None
    if S0 is not None:
        s0 = _f64(S0)
        if s0.shape != (B, H, dk, dv):
            raise ValueError("S0 shape mismatch")
    o = np.empty((B, H, L, dv))
    S_L = np.empty((B, H, dk, dv))
    rc = _lib().efla_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                    None if s0 is None else _ptr(s0), _ptr(o), _ptr(S_L),
                                    B, H, L, dk, dv, _euler(update), int(threads))
    if rc != 0:
        raise RuntimeError("oracle forward failed")
    return o, S_L


def decode(q, k, v, beta, S, threads: int = 0, update: str = "exact"):
    """One decode step.  Returns (o [N,H,dv], S_new [N,H,dk,dv]); S is not modified."""
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    S = _f64(S).copy()
    N, H, dk = k.shape
    dv = v.shape[-1]
    if q.shape != (N, H, dk) or v.shape != (N, H, dv) or beta.shape != (N, H) \
            or S.shape != (N, H, dk, dv):
        raise ValueError("shape mismatch")
    o = np.empty((N, H, dv))
    rc = _lib().efla_oracle_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S), _ptr(o),
                                   N, H, dk, dv, _euler(update), int(threads))
    if rc != 0:
        raise RuntimeError("oracle decode failed")
    return o, S


def alpha_grad(beta, lam, update: str = "exact"):
    """(d alpha / d beta, d alpha / d lambda) from the C oracle, elementwise (fp64)."""
    beta = _f64(beta)
    lam = _f64(lam)
    beta, lam = np.broadcast_arrays(beta, lam)
    db = np.empty(beta.shape)
    dl = np.empty(beta.shape)
    a = ctypes.c_double()
    b = ctypes.c_double()
    eu = _euler(update)
    for idx in np.ndindex(*beta.shape):
        _lib().efla_oracle_alpha_grad(float(beta[idx]), float(lam[idx]), eu, ctypes.byref(a),
                                      ctypes.byref(b))
        db[idx] = a.value
        dl[idx] = b.value
    return db, dl


def backward(q, k, v, beta, S0, dO, dS_L=None, threads: int = 0, update: str = "exact"):
    """Gradients through ``forward`` of a loss with dLoss/do = dO and
    dLoss/dS_L = dS_L (None: zero).  Returns (dq, dk, dv, dbeta, dS0) in fp64,
    shaped like q, k, v, beta and [B,H,dk,dv]; dS0 is returned even when S0 is
    None (the gradient with respect to the zero initial state)."""
    q, k, v, beta, dO = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(dO)
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    if q.shape != (B, H, L, dk) or v.shape != (B, H, L, dv) or beta.shape != (B, H, L) \
            or dO.shape != (B, H, L, dv):
        raise ValueError("shape mismatch")
    s0 = None if S0 is None else _f64(S0)
    dsl = None if dS_L is None else _f64(dS_L)
    for x in (s0, dsl):
        if x is not None and x.shape != (B, H, dk, dv):
            raise ValueError("state shape mismatch")
    dq = np.empty((B, H, L, dk))
    dk_ = np.empty((B, H, L, dk))
    dv_ = np.empty((B, H, L, dv))
    dbeta = np.empty((B, H, L))
    dS0 = np.empty((B, H, dk, dv))
    rc = _lib().efla_oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                     None if s0 is None else _ptr(s0), _ptr(dO),
                                     None if dsl is None else _ptr(dsl), _ptr(dq), _ptr(dk_),
                                     _ptr(dv_), _ptr(dbeta), _ptr(dS0), B, H, L, dk, dv,
                                     _euler(update), int(threads))
    if rc != 0:
        raise RuntimeError("oracle backward failed")
    return dq, dk_, dv_, dbeta, dS0
