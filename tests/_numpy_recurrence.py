"""An independent, dense numpy evaluation of the EFLA recurrence (fp64).

Used only to cross-check the C oracle's indexing.  It builds the full
d_k x d_k transition I - a k k^T and multiplies it out (O(d^3) per token),
which is a different route from the oracle's rank-1 evaluation.
"""
import numpy as np


def dense_forward(q, k, v, beta, S0=None):
    q, k, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta))
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, L, dv))
    SL = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for t in range(L):
                kt = k[b, h, t]
                lam = float(kt @ kt)
                bt = float(beta[b, h, t])
                a = bt if lam == 0.0 else (1.0 - np.exp(-bt * lam)) / lam
                P = np.eye(dk) - a * np.outer(kt, kt)
                S = P @ S + a * np.outer(kt, v[b, h, t])
                o[b, h, t] = S.T @ q[b, h, t]
            SL[b, h] = S
    return o, SL
