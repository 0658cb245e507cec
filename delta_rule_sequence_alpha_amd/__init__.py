"""EFLA (Exact Flow Linear Attention) forward operator and decode step on MI355X.

Torch-facing wrappers around the C ABI of libefla.so (include/efla.h).  torch
supplies device memory and the current stream; every step of the operator
runs in the library's HIP kernels.

  forward(q, k, v, beta, S0=None, chunk=64, path="auto", update="exact") -> (o, S_L)
  decode_step(q, k, v, beta, S, update="exact") -> o     (S updated in place)
  decode_step_indexed(q, k, v, beta, slots, S_pool) -> o  (pool entries slots[n] in place)
  forward_varlen(q, k, v, beta, cu_seqlens, S0=None, chunk=64) -> (o, S_L)
                                              packed sequences, [H, T, d] tensors
  coefficients(k, beta, update="exact") -> (alpha, lambda)   stage 1 of the staged path
update="euler" evaluates the explicit Euler step of the same ODE instead
(alpha = beta, the delta rule) on the same kernels.
  ut_transform(q, k, v, alpha, chunk) -> (W, U, A)   stage 2
  chunk_scan(q, k, W, U, A, S0, chunk) -> (o, S_L)   stage 3
  backward(q, k, v, beta, S0, d_o, dS_L=None, chunk=64, update="exact")
      -> (dq, dk, dv, dbeta, dS0)   gradients of a loss through forward
  efla(q, k, v, beta, S0=None, chunk=64, update="exact") -> (o, S_L)
      forward + backward as a torch.autograd.Function
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import (EFLA_BF16, EFLA_EULER, EFLA_EXACT, EFLA_F32, EFLA_PATH_AUTO, EFLA_PATH_FUSED,
                   EFLA_PATH_SEGMENTED, EFLA_PATH_STAGED, EflaError, LIB_PATH)

__all__ = ["forward", "forward_varlen", "decode_step", "decode_step_indexed", "coefficients", "ut_transform", "chunk_scan",
           "backward", "efla", "workspace_size", "varlen_workspace_size", "backward_workspace_size", "EflaError", "LIB_PATH"]

_PATHS = {"auto": EFLA_PATH_AUTO, "staged": EFLA_PATH_STAGED, "fused": EFLA_PATH_FUSED,
          "segmented": EFLA_PATH_SEGMENTED}
_UPDATES = {"exact": EFLA_EXACT, "euler": EFLA_EULER}


def _dt(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return EFLA_BF16
    if x.dtype == torch.float32:
        return EFLA_F32
    raise TypeError(f"unsupported dtype {x.dtype}; q, k, v must be bfloat16 or float32")


def _check(x: torch.Tensor, name: str, shape, dtype=None):
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if x.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {tuple(shape)}")
    if dtype is not None and x.dtype != dtype:
        raise TypeError(f"{name} has dtype {x.dtype}, expected {dtype}")


def _ptr(x):
    return None if x is None else x.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _raise(status: int, what: str):
    if status != _lib.EFLA_OK:
        raise EflaError(status, what)


def workspace_size(B, H, L, d_k, d_v, chunk, dtype, path="auto") -> int:
    dt = EFLA_BF16 if dtype == torch.bfloat16 else EFLA_F32
    return _lib.efla_forward_workspace_size_ex(B, H, L, d_k, d_v, chunk, dt, _PATHS[path])


def forward(q, k, v, beta, S0=None, chunk: int = 64, path: str = "auto", workspace=None,
            out=None, S_L=None, update: str = "exact", config=None):
    """Chunked EFLA forward.  q, k: [B,H,L,d_k]; v: [B,H,L,d_v]; beta: [B,H,L] fp32.

    Returns (o [B,H,L,d_v] in q's dtype, S_L [B,H,d_k,d_v] fp32).  ``workspace``
    (uint8, >= workspace_size bytes), ``out`` and ``S_L`` may be preallocated.
    ``config``: a launch configuration (dict with fused_scan_waves, scan_waves,
    bwd_scan_waves; None = the built-in one).
    """
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    dt = _dt(q)
    _check(q, "q", (B, H, L, dk), q.dtype)
    _check(k, "k", (B, H, L, dk), q.dtype)
    _check(v, "v", (B, H, L, dv), q.dtype)
    _check(beta, "beta", (B, H, L), torch.float32)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32)
    dev = q.device
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=q.dtype, device=dev)
    _check(out, "out", (B, H, L, dv), q.dtype)
    if S_L is None:
        S_L = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _check(S_L, "S_L", (B, H, dk, dv), torch.float32)
    p = _PATHS[path]
    need = _lib.efla_forward_workspace_size_ex(B, H, L, dk, dv, chunk, dt, p)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.efla_forward_config(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(out),
                                  _ptr(S_L), B, H, L, dk, dv, chunk, dt, _ptr(workspace), ws_bytes,
                                  p, _UPDATES[update], config, _stream(dev))
    _raise(st, "efla_forward_config")
    return out, S_L


def varlen_workspace_size(N, H, T, d_k, d_v, chunk, dtype, path="auto") -> int:
    """Bytes of device workspace forward_varlen needs on ``path``."""
    dt = EFLA_BF16 if dtype == torch.bfloat16 else EFLA_F32
    return _lib.efla_forward_varlen_workspace_size(N, H, T, d_k, d_v, chunk, dt, _PATHS[path])


def forward_varlen(q, k, v, beta, cu_seqlens, S0=None, chunk: int = 64, out=None, S_L=None,
                   update: str = "exact", path: str = "auto", workspace=None):
    """Packed sequences: q, k [H,T,d_k], v [H,T,d_v], beta [H,T]; cu_seqlens int32
    [N+1] on the device.  Returns (o [H,T,d_v], S_L [N,H,d_k,d_v] fp32).
    ``workspace`` (uint8, >= varlen_workspace_size bytes) may be preallocated."""
    H, T, dk = k.shape
    dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dt = _dt(q)
    _check(q, "q", (H, T, dk), q.dtype)
    _check(k, "k", (H, T, dk), q.dtype)
    _check(v, "v", (H, T, dv), q.dtype)
    _check(beta, "beta", (H, T), torch.float32)
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32)
    if S0 is not None:
        _check(S0, "S0", (N, H, dk, dv), torch.float32)
    if out is None:
        out = torch.empty((H, T, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", (H, T, dv), q.dtype)
    if S_L is None:
        S_L = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    _check(S_L, "S_L", (N, H, dk, dv), torch.float32)
    p = _PATHS[path]
    need = _lib.efla_forward_varlen_workspace_size(N, H, T, dk, dv, chunk, dt, p)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.efla_forward_varlen_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(cu_seqlens),
                                     _ptr(S0), _ptr(out), _ptr(S_L), N, H, T, dk, dv, chunk, dt,
                                     _UPDATES[update], p, _ptr(workspace), ws_bytes,
                                     _stream(q.device))
    _raise(st, "efla_forward_varlen_ex")
    return out, S_L


def decode_step(q, k, v, beta, S, out=None, update: str = "exact"):
    """One decode step, S [N,H,d_k,d_v] fp32 updated in place.  Returns o [N,H,d_v]."""
    N, H, dk = k.shape
    dv = v.shape[-1]
    dt = _dt(q)
    _check(q, "q", (N, H, dk), q.dtype)
    _check(k, "k", (N, H, dk), q.dtype)
    _check(v, "v", (N, H, dv), q.dtype)
    _check(beta, "beta", (N, H), torch.float32)
    _check(S, "S", (N, H, dk, dv), torch.float32)
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", (N, H, dv), q.dtype)
    st = _lib.efla_decode_step_update(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S), _ptr(out),
                                      N, H, dk, dv, dt, _UPDATES[update], _stream(q.device))
    _raise(st, "efla_decode_step_update")
    return out


def decode_step_indexed(q, k, v, beta, slots, S_pool, out=None, err=None, update: str = "exact"):
    """One decode step for N tokens whose states are pool entries: token n
    updates S_pool[slots[n]] ([P,H,d_k,d_v] fp32) in place.  slots: int32 [N]
    on the device, distinct, in [0, P).  err (int32 [1] on the device, or
    None): OR-ed with 1 / 2 for repeated / out-of-range slots, whose tokens
    are rejected (pool untouched, o = NaN).  Returns o [N,H,d_v]."""
    N, H, dk = k.shape
    dv = v.shape[-1]
    P = S_pool.shape[0]
    dt = _dt(q)
    _check(q, "q", (N, H, dk), q.dtype)
    _check(k, "k", (N, H, dk), q.dtype)
    _check(v, "v", (N, H, dv), q.dtype)
    _check(beta, "beta", (N, H), torch.float32)
    _check(slots, "slots", (N,), torch.int32)
    _check(S_pool, "S_pool", (P, H, dk, dv), torch.float32)
    if err is not None:
        _check(err, "err", (1,), torch.int32)
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", (N, H, dv), q.dtype)
    st = _lib.efla_decode_step_indexed(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(slots),
                                       _ptr(S_pool), _ptr(out), _ptr(err), N, H, P, dk, dv, dt,
                                       _UPDATES[update], _stream(q.device))
    _raise(st, "efla_decode_step_indexed")
    return out


def coefficients(k, beta, with_lambda: bool = True, update: str = "exact"):
    """Stage 1: per-token (alpha, lambda) in fp32, shaped like beta."""
    dk = k.shape[-1]
    n = beta.numel()
    _check(k, "k", tuple(beta.shape) + (dk,))
    _check(beta, "beta", tuple(beta.shape), torch.float32)
    alpha = torch.empty_like(beta)
    lam = torch.empty_like(beta) if with_lambda else None
    st = _lib.efla_coefficients_update(_ptr(k), _ptr(beta), _ptr(alpha), _ptr(lam), n, dk, _dt(k),
                                       _UPDATES[update], _stream(k.device))
    _raise(st, "efla_coefficients_update")
    return alpha, lam


def ut_transform(q, k, v, alpha, chunk: int = 64):
    """Stage 2: W [B,H,L,d_k], U [B,H,L,d_v], A [B,H,n_chunks,chunk,chunk] in q's dtype."""
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    _check(q, "q", (B, H, L, dk), q.dtype)
    _check(k, "k", (B, H, L, dk), q.dtype)
    _check(v, "v", (B, H, L, dv), q.dtype)
    _check(alpha, "alpha", (B, H, L), torch.float32)
    nch = (L + chunk - 1) // chunk
    W = torch.empty_like(k)
    U = torch.empty_like(v)
    A = torch.empty((B, H, nch, chunk, chunk), dtype=q.dtype, device=q.device)
    st = _lib.efla_ut_transform(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(W), _ptr(U), _ptr(A),
                                B, H, L, dk, dv, chunk, _dt(q), _stream(q.device))
    _raise(st, "efla_ut_transform")
    return W, U, A


def chunk_scan(q, k, W, U, A, S0=None, chunk: int = 64):
    """Stage 3: (o [B,H,L,d_v], S_L [B,H,d_k,d_v] fp32) from stage-2 outputs."""
    B, H, L, dk = k.shape
    dv = U.shape[-1]
    _check(W, "W", (B, H, L, dk), q.dtype)
    _check(U, "U", (B, H, L, dv), q.dtype)
    nch = (L + chunk - 1) // chunk
    _check(A, "A", (B, H, nch, chunk, chunk), q.dtype)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32)
    o = torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device)
    S_L = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    st = _lib.efla_chunk_scan(_ptr(q), _ptr(k), _ptr(W), _ptr(U), _ptr(A), _ptr(S0), _ptr(o),
                              _ptr(S_L), B, H, L, dk, dv, chunk, _dt(q), _stream(q.device))
    _raise(st, "efla_chunk_scan")
    return o, S_L


def backward_workspace_size(B, H, L, d_k, d_v, chunk, dtype) -> int:
    dt = EFLA_BF16 if dtype == torch.bfloat16 else EFLA_F32
    return _lib.efla_backward_workspace_size(B, H, L, d_k, d_v, chunk, dt)


def backward(q, k, v, beta, S0, d_o, dS_L=None, chunk: int = 64, update: str = "exact",
             workspace=None, want_dS0: bool = True, config=None):
    """Gradients of a loss through ``forward``: given d_o = dLoss/do and
    dS_L = dLoss/dS_L (None: zero), returns (dq, dk, dv, dbeta, dS0) with dq,
    dk, dv in q's dtype, dbeta and dS0 fp32 (dS0 None if not ``want_dS0``)."""
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    dt = _dt(q)
    _check(q, "q", (B, H, L, dk), q.dtype)
    _check(k, "k", (B, H, L, dk), q.dtype)
    _check(v, "v", (B, H, L, dv), q.dtype)
    _check(beta, "beta", (B, H, L), torch.float32)
    _check(d_o, "d_o", (B, H, L, dv), q.dtype)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32)
    if dS_L is not None:
        _check(dS_L, "dS_L", (B, H, dk, dv), torch.float32)
    dev = q.device
    dq = torch.empty_like(q)
    dkk = torch.empty_like(k)
    dvv = torch.empty_like(v)
    dbeta = torch.empty_like(beta)
    dS0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_dS0 else None
    need = _lib.efla_backward_workspace_size(B, H, L, dk, dv, chunk, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.efla_backward_config(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(d_o),
                                   _ptr(dS_L), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dbeta),
                                   _ptr(dS0), B, H, L, dk, dv, chunk, dt, _UPDATES[update], config,
                                   _ptr(workspace), ws_bytes, _stream(dev))
    _raise(st, "efla_backward_config")
    return dq, dkk, dvv, dbeta, dS0


class _EflaFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, beta, S0, chunk, update):
        o, S_L = forward(q, k, v, beta, S0, chunk=chunk, update=update)
        ctx.save_for_backward(q, k, v, beta, S0)
        ctx.chunk, ctx.update = chunk, update
        return o, S_L

    @staticmethod
    def backward(ctx, d_o, dS_L):
        q, k, v, beta, S0 = ctx.saved_tensors
        if d_o is None:
            d_o = torch.zeros_like(q[..., :1].expand(*q.shape[:-1], v.shape[-1]))
        d_o = d_o.contiguous()
        dS_L = None if dS_L is None else dS_L.contiguous()
        dq, dk, dv, dbeta, dS0 = backward(q, k, v, beta, S0, d_o, dS_L, chunk=ctx.chunk,
                                          update=ctx.update, want_dS0=S0 is not None)
        return dq, dk, dv, dbeta, dS0, None, None


def efla(q, k, v, beta, S0=None, chunk: int = 64, update: str = "exact"):
    """(o, S_L) = forward(...), differentiable in q, k, v, beta and S0."""
    return _EflaFunction.apply(q, k, v, beta, S0, chunk, update)
