"""Helpers shared by the GPU parity tests (error metric, tolerances, transfers)."""
import sys

import numpy as np
import torch

# Gates on err = max|gpu - oracle| / max|oracle|, per output tensor:
# fp32 inputs on fp32 MFMA, and bf16 inputs with fp32 accumulation.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(gpu, ref) -> float:
    g = gpu.detach().to("cpu", torch.float64).numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    den = np.max(np.abs(r)) if r.size else 0.0
    num = np.max(np.abs(g - r)) if r.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def dev(*xs, device="cuda"):
    out = tuple(None if x is None else x.to(device).contiguous() for x in xs)
    return out if len(out) > 1 else out[0]


def note(msg: str):
    """Name the case before a GPU step, flushed, so a fault points at it."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)
