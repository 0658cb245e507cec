"""ctypes binding of libefla.so: the C ABI of include/efla.h (and the peak
reference kernels of include/efla_peaks.h), name for name.

Argument marshalling only.  Every step of the operator runs in the HIP
kernels of libefla.so; if the library is missing this module raises instead
of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libefla.so")

EFLA_F32, EFLA_BF16 = 0, 1
EFLA_OK, EFLA_ERR_INVALID_ARG, EFLA_ERR_UNSUPPORTED, EFLA_ERR_WORKSPACE, EFLA_ERR_HIP = range(5)
EFLA_PATH_AUTO, EFLA_PATH_STAGED, EFLA_PATH_FUSED, EFLA_PATH_SEGMENTED = 0, 1, 2, 3
EFLA_EXACT, EFLA_EULER = 0, 1

# (name, restype, argtypes) of every exported symbol, in header order.
_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_long
_S = ctypes.c_size_t
SIGNATURES = [
    ("efla_forward_path", _I, [_I] * 7),
    ("efla_status_string", ctypes.c_char_p, [_I]),
    ("efla_forward_workspace_size", _S, [_I, _I, _I, _I, _I, _I, _I]),
    ("efla_forward_workspace_size_ex", _S, [_I, _I, _I, _I, _I, _I, _I, _I]),
    ("efla_forward", _I, [_P] * 7 + [_I] * 7 + [_P, _S, _P]),
    ("efla_forward_ex", _I, [_P] * 7 + [_I] * 7 + [_P, _S, _I, _P]),
    ("efla_forward_varlen", _I, [_P] * 8 + [_I] * 8 + [_P]),
    ("efla_forward_varlen_workspace_size", _S, [_I] * 8),
    ("efla_forward_varlen_ex", _I, [_P] * 8 + [_I] * 9 + [_P, _S, _P]),
    ("efla_forward_update", _I, [_P] * 7 + [_I] * 7 + [_P, _S, _I, _I, _P]),
    ("efla_forward_config", _I, [_P] * 7 + [_I] * 7 + [_P, _S, _I, _I, _P, _P]),
    ("efla_forward_noalloc", _I, [_P] * 7 + [_I] * 7 + [_I, _I, _P]),
    ("efla_decode_step", _I, [_P] * 6 + [_I] * 5 + [_P]),
    ("efla_decode_step_update", _I, [_P] * 6 + [_I] * 6 + [_P]),
    ("efla_decode_step_indexed", _I, [_P] * 8 + [_I] * 7 + [_P]),
    ("efla_coefficients", _I, [_P] * 4 + [_L, _I, _I, _P]),
    ("efla_coefficients_update", _I, [_P] * 4 + [_L, _I, _I, _I, _P]),
    ("efla_ut_transform", _I, [_P] * 7 + [_I] * 7 + [_P]),
    ("efla_chunk_scan", _I, [_P] * 8 + [_I] * 7 + [_P]),
    ("efla_backward_workspace_size", _S, [_I] * 7),
    ("efla_backward", _I, [_P] * 12 + [_I] * 8 + [_P, _S, _P]),
    ("efla_backward_config", _I, [_P] * 12 + [_I] * 8 + [_P, _P, _S, _P]),
    # include/efla_peaks.h
    ("efla_peak_copy", _I, [_P, _P, _S, _P]),
    ("efla_peak_mfma", _I, [_P, _I, _I, _I, _P, _P]),
]


class LaunchConfig(ctypes.Structure):
    """efla_launch_config_t: 0 in a field takes the library's built-in choice."""
    _fields_ = [("fused_scan_waves", _I), ("scan_waves", _I), ("bwd_scan_waves", _I)]


def launch_config(cfg) -> LaunchConfig | None:
    """A LaunchConfig from None, a LaunchConfig or a dict of its fields."""
    if cfg is None or isinstance(cfg, LaunchConfig):
        return cfg
    return LaunchConfig(**cfg)


_lib = None


class EflaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


def lib() -> ctypes.CDLL:
    """Load libefla.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m delta_rule_sequence_alpha_amd.build)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(s: int) -> str:
    return lib().efla_status_string(int(s)).decode()


def _call(name: str, *args) -> int:
    return int(getattr(lib(), name)(*args))


def efla_forward_path(B, H, L, dk, dv, chunk, dt) -> int:
    return int(lib().efla_forward_path(B, H, L, dk, dv, chunk, dt))


def efla_status_string(s: int) -> str:
    return status_string(s)


def efla_forward_workspace_size(B, H, L, dk, dv, chunk, dt) -> int:
    return int(lib().efla_forward_workspace_size(B, H, L, dk, dv, chunk, dt))


def efla_forward_workspace_size_ex(B, H, L, dk, dv, chunk, dt, path) -> int:
    return int(lib().efla_forward_workspace_size_ex(B, H, L, dk, dv, chunk, dt, path))


def efla_forward(q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt, ws, ws_bytes, stream) -> int:
    return _call("efla_forward", q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt, ws,
                 ws_bytes, stream)


def efla_forward_ex(q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt, ws, ws_bytes, path,
                    stream) -> int:
    return _call("efla_forward_ex", q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt, ws,
                 ws_bytes, path, stream)


def efla_forward_update(q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt, ws, ws_bytes,
                        path, update, stream) -> int:
    return _call("efla_forward_update", q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt, ws,
                 ws_bytes, path, update, stream)


def efla_forward_config(q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt, ws, ws_bytes,
                        path, update, config, stream) -> int:
    cfg = launch_config(config)
    return _call("efla_forward_config", q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt, ws,
                 ws_bytes, path, update, None if cfg is None else ctypes.byref(cfg), stream)


def efla_forward_noalloc(q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt, path, update,
                         stream) -> int:
    return _call("efla_forward_noalloc", q, k, v, beta, S0, o, S_L, B, H, L, dk, dv, chunk, dt,
                 path, update, stream)


NOALLOC_SCRATCH_BYTES = 64 << 20   # EFLA_NOALLOC_SCRATCH_BYTES


def efla_forward_varlen(q, k, v, beta, cu_seqlens, S0, o, S_L, N, H, T, dk, dv, chunk, dt, update,
                        stream) -> int:
    return _call("efla_forward_varlen", q, k, v, beta, cu_seqlens, S0, o, S_L, N, H, T, dk, dv,
                 chunk, dt, update, stream)


def efla_forward_varlen_workspace_size(N, H, T, dk, dv, chunk, dt, path) -> int:
    return int(lib().efla_forward_varlen_workspace_size(N, H, T, dk, dv, chunk, dt, path))


def efla_forward_varlen_ex(q, k, v, beta, cu_seqlens, S0, o, S_L, N, H, T, dk, dv, chunk, dt,
                           update, path, ws, ws_bytes, stream) -> int:
    return _call("efla_forward_varlen_ex", q, k, v, beta, cu_seqlens, S0, o, S_L, N, H, T, dk, dv,
                 chunk, dt, update, path, ws, ws_bytes, stream)


def efla_decode_step(q, k, v, beta, S, o, N, H, dk, dv, dt, stream) -> int:
    return _call("efla_decode_step", q, k, v, beta, S, o, N, H, dk, dv, dt, stream)


def efla_decode_step_update(q, k, v, beta, S, o, N, H, dk, dv, dt, update, stream) -> int:
    return _call("efla_decode_step_update", q, k, v, beta, S, o, N, H, dk, dv, dt, update, stream)


def efla_decode_step_indexed(q, k, v, beta, slots, S_pool, o, err, N, H, P, dk, dv, dt, update,
                             stream) -> int:
    return _call("efla_decode_step_indexed", q, k, v, beta, slots, S_pool, o, err, N, H, P, dk, dv,
                 dt, update, stream)


def efla_coefficients(k, beta, alpha, lam, n_tokens, dk, dt, stream) -> int:
    return _call("efla_coefficients", k, beta, alpha, lam, n_tokens, dk, dt, stream)


def efla_coefficients_update(k, beta, alpha, lam, n_tokens, dk, dt, update, stream) -> int:
    return _call("efla_coefficients_update", k, beta, alpha, lam, n_tokens, dk, dt, update, stream)


def efla_ut_transform(q, k, v, alpha, w, u, a_qk, B, H, L, dk, dv, chunk, dt, stream) -> int:
    return _call("efla_ut_transform", q, k, v, alpha, w, u, a_qk, B, H, L, dk, dv, chunk, dt,
                 stream)


def efla_chunk_scan(q, k, w, u, a_qk, S0, o, S_L, B, H, L, dk, dv, chunk, dt, stream) -> int:
    return _call("efla_chunk_scan", q, k, w, u, a_qk, S0, o, S_L, B, H, L, dk, dv, chunk, dt,
                 stream)


def efla_backward_workspace_size(B, H, L, dk, dv, chunk, dt) -> int:
    return int(lib().efla_backward_workspace_size(B, H, L, dk, dv, chunk, dt))


def efla_backward(q, k, v, beta, S0, d_o, dS_L, dq, dk_, dv_, dbeta, dS0, B, H, L, dk, dv, chunk,
                  dt, update, ws, ws_bytes, stream) -> int:
    return _call("efla_backward", q, k, v, beta, S0, d_o, dS_L, dq, dk_, dv_, dbeta, dS0, B, H, L,
                 dk, dv, chunk, dt, update, ws, ws_bytes, stream)


def efla_backward_config(q, k, v, beta, S0, d_o, dS_L, dq, dk_, dv_, dbeta, dS0, B, H, L, dk, dv,
                         chunk, dt, update, config, ws, ws_bytes, stream) -> int:
    cfg = launch_config(config)
    return _call("efla_backward_config", q, k, v, beta, S0, d_o, dS_L, dq, dk_, dv_, dbeta, dS0, B,
                 H, L, dk, dv, chunk, dt, update, None if cfg is None else ctypes.byref(cfg), ws,
                 ws_bytes, stream)


def efla_peak_copy(src, dst, nbytes, stream) -> int:
    return _call("efla_peak_copy", src, dst, nbytes, stream)


def efla_peak_mfma(sink, blocks, iters, dt, stream) -> tuple:
    """(status, flops of one launch)."""
    fl = ctypes.c_double(0.0)
    st = _call("efla_peak_mfma", sink, blocks, iters, dt, ctypes.byref(fl), stream)
    return st, fl.value
