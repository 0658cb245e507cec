"""Seeded synthetic inputs for the EFLA forward operator and decode step.

This module only draws random numbers and casts them to the storage dtype.  It
holds none of the method's arithmetic (no coefficient, no state update, no
readout), so both the fp64 oracle and the HIP path may consume what it makes.

Workloads (shapes, value distributions and structure follow the five workloads
the operator is measured on; the pages themselves give no model shapes, see
"Exact Flow Linear Attention: Exact Solution from Continuous-Time Dynamics",
Technical Summary, Experimental Results):

  tiny-f32         B=1  H=1  L=64     d=16  C=16  fp32
  lm340m-bf16      B=8  H=8  L=2048   d=128 C=64  bf16 storage
  lm1.3b-bf16      B=4  H=16 L=4096   d=128 C=64  bf16 storage, random S0
  long-stiff-f32   B=1  H=16 L=65536  d=128 C=64  fp32, key spikes x10
  decode-f32       N=256 H=16 d=128, fp32 state, 1000 single-token steps

Draw order for a forward workload, from one numpy PCG64 stream seeded with
``seed``: q, k (direction, then norm), v, beta, spike mask, S0.  ``N(0, s)``
means standard deviation ``s``; ``LogUniform[a, b]`` is ``exp(U(ln a, ln b))``;
a direction uniform on the sphere is ``g / |g|`` with ``g ~ N(0, I)``.  The
spike mask is one Bernoulli(0.05) draw per (batch, position), shared by all
heads.  bf16 tensors are the round-to-nearest-even cast of the fp32 draw.

Packed (varlen) batches: ``varlen_lengths`` splits a token total at sorted
uniform cut points; ``varlen_inputs`` draws one [1, H, T, d] batch with a
recipe and returns it as [H, T, d] with the cumulative offsets, and per-
sequence initial states from ``default_rng([seed, 1])``.
Decode: the state is drawn from ``default_rng([seed, 0])``; the tokens of step
``s`` (s = 0, 1, ...) come from ``default_rng([seed, s + 1])`` in the order q, k,
v, beta.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = [
    "ForwardWorkload",
    "DecodeWorkload",
    "FORWARD_WORKLOADS",
    "DECODE_WORKLOADS",
    "forward_inputs",
    "decode_state",
    "decode_tokens",
    "varlen_lengths",
    "varlen_inputs",
    "output_grads",
]


@dataclasses.dataclass(frozen=True)
class ForwardWorkload:
    name: str
    B: int
    H: int
    L: int
    d_k: int
    d_v: int
    chunk: int
    dtype: str            # storage dtype of q, k, v, o: "f32" or "bf16"
    recipe: str           # value-distribution recipe, see forward_inputs()

    def with_(self, **kw) -> "ForwardWorkload":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    N: int
    H: int
    d_k: int
    d_v: int
    steps: int
    dtype: str


FORWARD_WORKLOADS = {
    w.name: w
    for w in [
        ForwardWorkload("tiny-f32", 1, 1, 64, 16, 16, 16, "f32", "tiny"),
        ForwardWorkload("lm340m-bf16", 8, 8, 2048, 128, 128, 64, "bf16", "lm340m"),
        ForwardWorkload("lm1.3b-bf16", 4, 16, 4096, 128, 128, 64, "bf16", "lm1.3b"),
        ForwardWorkload("long-stiff-f32", 1, 16, 65536, 128, 128, 64, "f32", "stiff"),
    ]
}

DECODE_WORKLOADS = {
    w.name: w for w in [DecodeWorkload("decode-f32", 256, 16, 128, 128, 1000, "f32")]
}


def _normal(rng: np.random.Generator, shape, std=1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _sphere(rng: np.random.Generator, shape) -> np.ndarray:
    g = rng.standard_normal(size=shape, dtype=np.float64)
    n = np.sqrt(np.sum(g * g, axis=-1, keepdims=True))
    return (g / n).astype(np.float32)


def _sigmoid_normal(rng: np.random.Generator, shape) -> np.ndarray:
    z = rng.standard_normal(size=shape, dtype=np.float64)
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def _log_uniform(rng: np.random.Generator, shape, lo, hi) -> np.ndarray:
    return np.exp(rng.uniform(math.log(lo), math.log(hi), size=shape)).astype(np.float32)


def _store(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(f"unknown storage dtype {dtype!r}")


def forward_inputs(w: ForwardWorkload, seed: int = 0):
    """Return (q, k, v, beta, S0) as CPU torch tensors.

    q, k: [B,H,L,d_k] and v: [B,H,L,d_v] in the workload's storage dtype;
    beta: [B,H,L] fp32; S0: [B,H,d_k,d_v] fp32, or None for the zero state.
    """
    rng = np.random.default_rng(seed)
    B, H, L, dk, dv = w.B, w.H, w.L, w.d_k, w.d_v
    S0 = None
    if w.recipe == "tiny":
        q = _normal(rng, (B, H, L, dk))
        k = _sphere(rng, (B, H, L, dk)) * _log_uniform(rng, (B, H, L, 1), 0.1, 4.0)
        v = _normal(rng, (B, H, L, dv))
        beta = rng.uniform(0.0, 1.0, size=(B, H, L)).astype(np.float32)
    elif w.recipe == "lm340m":
        q = _normal(rng, (B, H, L, dk), 1.0 / math.sqrt(dk))
        k = _sphere(rng, (B, H, L, dk)) * rng.uniform(0.5, 2.0, size=(B, H, L, 1)).astype(np.float32)
        v = _normal(rng, (B, H, L, dv))
        beta = _sigmoid_normal(rng, (B, H, L))
    elif w.recipe == "lm1.3b":
        q = _normal(rng, (B, H, L, dk), 1.0 / math.sqrt(dk))
        k = _normal(rng, (B, H, L, dk), 1.0 / math.sqrt(dk))
        v = _normal(rng, (B, H, L, dv))
        beta = _sigmoid_normal(rng, (B, H, L))
        S0 = _normal(rng, (B, H, dk, dv), 0.02)
    elif w.recipe == "stiff":
        q = _normal(rng, (B, H, L, dk))
        k = _sphere(rng, (B, H, L, dk)) * _log_uniform(rng, (B, H, L, 1), 0.1, 10.0)
        v = _normal(rng, (B, H, L, dv))
        beta = rng.uniform(0.0, 5.0, size=(B, H, L)).astype(np.float32)
        spike = rng.random(size=(B, 1, L, 1)) < 0.05
        k = np.where(spike, k * np.float32(10.0), k).astype(np.float32)
    else:
        raise ValueError(f"unknown recipe {w.recipe!r}")
    return (
        _store(q, w.dtype),
        _store(k, w.dtype),
        _store(v, w.dtype),
        torch.from_numpy(np.ascontiguousarray(beta, dtype=np.float32)),
        None if S0 is None else torch.from_numpy(np.ascontiguousarray(S0)),
    )


def decode_state(w: DecodeWorkload, seed: int = 0, n_seq: int | None = None) -> torch.Tensor:
    """Initial decode state S [N,H,d_k,d_v] fp32 ~ N(0, std 0.05).

    ``n_seq`` keeps only the first ``n_seq`` sequences of the same draw.
    """
    rng = np.random.default_rng([seed, 0])
    S = _normal(rng, (w.N, w.H, w.d_k, w.d_v), 0.05)
    if n_seq is not None:
        S = S[:n_seq]
    return torch.from_numpy(np.ascontiguousarray(S))


def decode_tokens(w: DecodeWorkload, step: int, seed: int = 0, n_seq: int | None = None):
    """Tokens of decode step ``step``: q, k [N,H,d_k], v [N,H,d_v], beta [N,H].

    q, v ~ N(0,1); k ~ N(0,1)/sqrt(d_k); beta = sigmoid(N(0,1)).
    """
    rng = np.random.default_rng([seed, step + 1])
    N, H, dk, dv = w.N, w.H, w.d_k, w.d_v
    q = _normal(rng, (N, H, dk))
    k = _normal(rng, (N, H, dk), 1.0 / math.sqrt(dk))
    v = _normal(rng, (N, H, dv))
    beta = _sigmoid_normal(rng, (N, H))
    if n_seq is not None:
        q, k, v, beta = q[:n_seq], k[:n_seq], v[:n_seq], beta[:n_seq]
    return (_store(q, w.dtype), _store(k, w.dtype), _store(v, w.dtype),
            torch.from_numpy(np.ascontiguousarray(beta)))


def varlen_lengths(n: int, total: int, seed: int = 0, min_len: int = 0) -> list:
    """n sequence lengths (>= min_len) summing to ``total``: a uniform random
    split of the remaining tokens (sorted cut points), so short, long and
    empty sequences all occur."""
    rng = np.random.default_rng([seed, 7])
    rest = total - n * min_len
    if rest < 0:
        raise ValueError("total too small for n * min_len")
    cuts = np.sort(rng.integers(0, rest + 1, size=n - 1))
    parts = np.diff(np.concatenate([[0], cuts, [rest]]))
    return [int(p) + min_len for p in parts]


def varlen_inputs(w: ForwardWorkload, lengths, seed: int = 0):
    """Packed sequences for the varlen forward, values drawn with recipe
    ``w.recipe`` (the workload's B and L are ignored; its H, d_k, d_v, dtype
    are used).  Returns (q, k [H,T,d_k], v [H,T,d_v], beta [H,T], cu_seqlens
    int32 [N+1], S0 [N,H,d_k,d_v] fp32 or None) as CPU tensors; T = sum of
    lengths, sequence n at tokens [cu_seqlens[n], cu_seqlens[n+1])."""
    T = int(sum(lengths))
    q, k, v, beta, S0 = forward_inputs(w.with_(B=1, L=T), seed=seed)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    S0n = None
    if S0 is not None:
        rng = np.random.default_rng([seed, 1])
        S0n = torch.from_numpy(_normal(rng, (len(lengths), w.H, w.d_k, w.d_v), 0.02))
    return q[0], k[0], v[0], beta[0], cu, S0n


def output_grads(w: ForwardWorkload, seed: int = 0, with_dS_L: bool = True):
    """Upstream gradients for a backward pass: (dO, dS_L) as CPU tensors.

    dO [B,H,L,d_v] ~ N(0,1)/sqrt(L) in the storage dtype (a loss averaged
    over tokens); dS_L [B,H,d_k,d_v] fp32 ~ N(0, std 0.02), or None.
    Drawn from their own stream (seed, 1), independent of the inputs.
    """
    rng = np.random.default_rng([seed, 1])
    B, H, L, dk, dv = w.B, w.H, w.L, w.d_k, w.d_v
    dO = _normal(rng, (B, H, L, dv), 1.0 / math.sqrt(max(L, 1)))
    dSL = _normal(rng, (B, H, dk, dv), 0.02) if with_dS_L else None
    return _store(dO, w.dtype), None if dSL is None else torch.from_numpy(np.ascontiguousarray(dSL))
