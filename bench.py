#!/usr/bin/env python3
"""Benchmark of the EFLA chunked forward (and the decode step) on one MI355X.

A step is one pass of the whole forward (coefficients, UT transform, state
scan -- or the fused kernel) over one batch of the lm1.3b-bf16 workload
(B=4, H=16, L=4096, d_k=d_v=128, chunk 64, bf16 inputs, fp32 state, random
S0), with every input resident in HBM before the timed region.  Prints one
JSON line.  The decode step (256 sequences x 16 heads, d=128, fp32 state) is
timed in the same run and reported under "decode".

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload lm1.3b-bf16]
                  [--path auto|staged|fused|segmented] [--no-cpu-baseline] [--no-decode]
                  [--no-compare] [--no-backward] [--no-cold] [--no-peaks]

The fused path is also timed with the Euler update (alpha = beta) and both
kernel times are reported under "update_compare"; a packed (varlen) batch of
the same token count is timed under "varlen" (and one of the long-stiff-f32
token count, on the segmented path, under "varlen_f32"), and the backward pass (dq, dk,
dv, dbeta, dS0 given dO and dS_L) of the same workload under "backward".
"call_ms" has per-call median/p10/p90 times, warm and cold (1 GiB written
between calls); "decode_512" the decode step with a state twice the Infinity
Cache; "configs" the lm340m-bf16 and long-stiff-f32 forwards, each with its
roofline, per-call times and oracle baseline; "measured_peaks" what the
library's reference copy and MFMA-loop kernels reach (include/efla_peaks.h),
against which every roofline also states a fraction.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import delta_rule_sequence_alpha_amd as efla  # noqa: E402
from delta_rule_sequence_alpha_amd import _lib  # noqa: E402
import efla_workloads as wl  # noqa: E402

METRIC = "EFLA chunked fwd tokens/s + % bf16 MFMA peak; decode-step state GB/s"
HBM_PEAK = 8.0e12                      # B/s, MI355X HBM3E
MFMA_PEAK = {"bf16": 2.5e15, "f32": 157.3e12}   # dense FLOP/s
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "delta_rule_sequence_alpha_amd", "csrc")


# --- algorithmic work (per token-head unless stated) ------------------------

def flops_per_token(dk, dv, C):
    """Whole forward: W S, Q S, K^T E (2 dk dv each), tril(QK^T) E (C dv),
    Gram and Q K^T lower triangles (C dk each), W = T K (C dk), U = T V (C dv),
    T by substitution (C^2/3)."""
    return 6 * dk * dv + C * (3 * dk + 2 * dv) + C * C / 3.0


def stage_work(w, esz):
    """(flops, bytes) per launch of each kernel of the staged path: minimal
    bytes each kernel must move (inputs read once, outputs written once)."""
    B, H, L, dk, dv, C = w.B, w.H, w.L, w.d_k, w.d_v, w.chunk
    n = B * H * L
    nch = B * H * ((L + C - 1) // C)
    s0 = 4 * B * H * dk * dv
    coef = (2 * dk * n, n * (dk * esz + 4 + 4))
    ut = ((C * (3 * dk + dv) + C * C / 3.0) * n,
          n * ((2 * dk + dv) * esz + 4) + n * (dk + dv) * esz + nch * C * C * esz)
    scan = ((6 * dk * dv + C * dv) * n,
            n * (2 * dk + dk + dv) * esz + nch * C * C * esz + n * dv * esz + 2 * s0)
    return {"coef": coef, "ut": ut, "scan": scan}


def fused_work(w, esz, has_s0):
    B, H, L, dk, dv, C = w.B, w.H, w.L, w.d_k, w.d_v, w.chunk
    n = B * H * L
    s = 4 * B * H * dk * dv
    return (flops_per_token(dk, dv, C) * n,
            n * ((2 * dk + dv) * esz + 4) + n * dv * esz + s * (2 if has_s0 else 1))


def source_hash(name: str) -> str:
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(kernel: str, workload: str, src: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken on the current source of the kernel; else None."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_h = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_h or not m_b or m_h.group(1) != source_hash(src):
        return None
    return float(m_b.group(1))


# --- timing helpers ---------------------------------------------------------

class Timer:
    """HIP events recorded on the stream the kernels are launched on."""

    def __init__(self, stream, names):
        self.stream = stream
        self.names = names
        self.ms = {n: [] for n in names}

    def marks(self):
        return [torch.cuda.Event(enable_timing=True) for _ in range(len(self.names) + 1)]

    def record(self, ev):
        ev.record(self.stream)

    def collect(self, pending):
        for evs in pending:
            for i, n in enumerate(self.names):
                self.ms[n].append(evs[i].elapsed_time(evs[i + 1]))

    def mean(self, n):
        v = self.ms[n]
        return sum(v) / len(v)


def bench_forward(args, w, dev):
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=0)
    host = (q, k, v, beta, S0)
    qd, kd, vd, bd = (x.to(dev) for x in (q, k, v, beta))
    s0d = None if S0 is None else S0.to(dev)
    dt = _lib.EFLA_BF16 if w.dtype == "bf16" else _lib.EFLA_F32
    esz = 2 if w.dtype == "bf16" else 4
    path = args.path
    if path == "auto":   # the library's own choice for this shape
        path = {_lib.EFLA_PATH_FUSED: "fused", _lib.EFLA_PATH_STAGED: "staged",
                _lib.EFLA_PATH_SEGMENTED: "segmented"}[
            _lib.efla_forward_path(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, dt)]
    pcode = {"staged": _lib.EFLA_PATH_STAGED, "fused": _lib.EFLA_PATH_FUSED,
             "segmented": _lib.EFLA_PATH_SEGMENTED}[path]
    B, H, L, dk, dv, C = w.B, w.H, w.L, w.d_k, w.d_v, w.chunk
    o = torch.empty((B, H, L, dv), dtype=qd.dtype, device=dev)
    S_L = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    if path == "staged":
        nch = (L + C - 1) // C
        alpha = torch.empty((B, H, L), dtype=torch.float32, device=dev)
        W = torch.empty_like(kd)
        U = torch.empty_like(vd)
        A = torch.empty((B, H, nch, C, C), dtype=qd.dtype, device=dev)
        names = ["coef", "ut", "scan"]

        def step(ev, timer):
            p = lambda x: None if x is None else x.data_ptr()  # noqa: E731
            timer.record(ev[0])
            st = _lib.efla_coefficients(p(kd), p(bd), p(alpha), None, B * H * L, dk, dt, sp)
            timer.record(ev[1])
            st |= _lib.efla_ut_transform(p(qd), p(kd), p(vd), p(alpha), p(W), p(U), p(A), B, H, L,
                                         dk, dv, C, dt, sp)
            timer.record(ev[2])
            st |= _lib.efla_chunk_scan(p(qd), p(kd), p(W), p(U), p(A), p(s0d), p(o), p(S_L), B, H,
                                       L, dk, dv, C, dt, sp)
            timer.record(ev[3])
            if st:
                raise RuntimeError("staged forward failed")
        work = stage_work(w, esz)
        srcs = {"coef": "coef_decode.hip", "ut": "ut_transform.hip", "scan": "chunk_scan.hip"}
    else:
        need = _lib.efla_forward_workspace_size_ex(B, H, L, dk, dv, C, dt, pcode)
        update = [_lib.EFLA_EXACT]
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        names = [path]

        def step(ev, timer):   # one kernel: timed over the whole region (ev, timer unused)
            p = lambda x: None if x is None else x.data_ptr()  # noqa: E731
            st = _lib.efla_forward_update(p(qd), p(kd), p(vd), p(bd), p(s0d), p(o), p(S_L), B,
                                          H, L, dk, dv, C, dt, p(ws), need, pcode, update[0], sp)
            if st:
                raise RuntimeError(f"fused forward failed: {_lib.status_string(st)}")
        work = {path: fused_work(w, esz, S0 is not None)}
        srcs = {path: "fused_forward.hip" if path == "fused" else "chunk_scan.hip"}

    def timed(k_steps):
        """Warmup, then k_steps steps between HIP events on the launch stream.
        Returns (wall seconds, per-kernel mean ms).  The single fused kernel is
        timed over the whole region (its mean launch duration); the staged
        kernels each get an event pair per launch."""
        timer = Timer(stream, names)
        for _ in range(args.warmup):
            step(timer.marks(), timer)
        torch.cuda.synchronize()
        pending = []
        r0 = torch.cuda.Event(enable_timing=True)
        r1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        r0.record(stream)
        for _ in range(k_steps):
            ev = timer.marks() if path == "staged" else None
            step(ev, timer)
            pending.append(ev)
        r1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if path == "staged":
            timer.collect(pending)
            return wall, {n: timer.mean(n) for n in names}
        return wall, {path: r0.elapsed_time(r1) / k_steps}

    elapsed, per_kernel = timed(args.steps)

    # Per-call times (an event pair around each call): warm, back to back; and
    # cold, with a 1 GiB buffer written between calls so that neither the L2s
    # nor the 256 MiB Infinity Cache hold any input.
    def per_call(n, cold):
        scratch = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev) if cold else None
        timer = Timer(stream, names)
        ms = []
        for i in range(n):
            if cold:
                scratch.fill_(i & 0xff)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step(timer.marks() if path == "staged" else None, timer)
            b.record(stream)
            ms.append((a, b))
        torch.cuda.synchronize()
        t = sorted(x.elapsed_time(y) for x, y in ms)
        pick = lambda f: t[min(len(t) - 1, int(f * (len(t) - 1) + 0.5))]  # noqa: E731
        return {"calls": n, "median_ms": pick(0.5), "p10_ms": pick(0.1), "p90_ms": pick(0.9)}
    call_stats = {"warm": per_call(max(args.steps, 10), False)}
    if not args.no_cold:
        call_stats["cold"] = per_call(10, True)

    # The same kernel with the explicit Euler step (alpha = beta, the delta
    # rule the exact flow is compared against), timed the same way.
    compare = None
    if path == "fused" and not args.no_compare:
        update[0] = _lib.EFLA_EULER
        _, eu = timed(args.steps)
        update[0] = _lib.EFLA_EXACT
        ex_ms, eu_ms = per_kernel["fused"], eu["fused"]
        compare = {"exact_kernel_ms": ex_ms, "euler_kernel_ms": eu_ms,
                   "exact_over_euler_time": ex_ms / eu_ms,
                   "note": "same fused kernel, alpha from the exact flow vs alpha = beta"}

    ms_step = elapsed * 1e3 / args.steps
    tokens = B * L
    F = flops_per_token(dk, dv, C) * B * H * L
    peak = MFMA_PEAK[w.dtype]
    dom = max(per_kernel, key=per_kernel.get)
    fl, by = work[dom]
    t_dom = per_kernel[dom] * 1e-3
    ridge = peak / HBM_PEAK
    bound = "mfma" if fl / by >= ridge else "hbm"
    traffic = read_traffic(dom, w.name, srcs[dom])
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": by / t_dom / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": fl / t_dom / 1e12, "peak": peak / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic
    roof["kernel"] = dom
    roof["kernel_ms"] = per_kernel[dom]
    roof["algorithmic_flops"] = fl
    roof["algorithmic_bytes"] = by
    res = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "L": L, "d_k": dk, "d_v": dv, "chunk": C,
                   "path": path, "S0": S0 is not None},
        "tflops": F / (ms_step * 1e-3) / 1e12,
        "mfma_frac": F / (ms_step * 1e-3) / peak,
        "flops_per_token_head": flops_per_token(dk, dv, C),
        "kernel_ms": per_kernel,
        "roofline": roof,
        "call_ms": call_stats,
    }
    if compare is not None:
        res["update_compare"] = compare
    return res, host


def bench_decode(args, dev, n_distinct=8, n_seq=None):
    w = wl.DECODE_WORKLOADS["decode-f32"]
    if n_seq is not None:
        w = dataclasses.replace(w, N=n_seq)
    S = wl.decode_state(w, seed=0).to(dev)
    toks = []
    for s in range(n_distinct):
        toks.append(tuple(x.to(dev) for x in wl.decode_tokens(w, s, seed=0)))
    o = torch.empty((w.N, w.H, w.d_v), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    p = lambda x: x.data_ptr()  # noqa: E731

    def step(i):
        q, k, v, beta = toks[i % n_distinct]
        st = _lib.efla_decode_step(p(q), p(k), p(v), p(beta), p(S), p(o), w.N, w.H, w.d_k, w.d_v,
                                   _lib.EFLA_F32, sp)
        if st:
            raise RuntimeError("decode failed")

    # the workload's 1000 steps; --decode-only (counter runs) takes --steps
    n_steps = args.steps if args.decode_only else w.steps
    for i in range(max(10, args.warmup)):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n_steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n_steps
    nh = w.N * w.H
    by = nh * (2 * w.d_k * w.d_v * 4 + (2 * w.d_k + 2 * w.d_v) * 4 + 4)
    return {"workload": w.name, "N": w.N, "H": w.H, "d_k": w.d_k, "d_v": w.d_v,
            "steps": n_steps, "ms_per_step": ms, "GB_s": by / (ms * 1e-3) / 1e9,
            "hbm_frac": by / (ms * 1e-3) / HBM_PEAK, "algorithmic_bytes": by,
            "note": f"{n_distinct} distinct token sets cycled over the steps; the state is "
                    f"{nh * w.d_k * w.d_v * 4} B against the 256 MiB Infinity Cache"}


def bench_varlen(args, dev, name="lm1.3b-bf16", n_seq=16):
    """Packed sequences: the workload's token count per head (B x L) split at
    random into n_seq sequences, its H heads, on the path AUTO takes (the
    fused kernel for bf16, the segmented scan for the long fp32 case)."""
    w = wl.FORWARD_WORKLOADS[name]
    lengths = wl.varlen_lengths(n_seq, w.B * w.L, seed=0)
    q, k, v, beta, cu, S0 = wl.varlen_inputs(w, lengths, seed=0)
    qd, kd, vd, bd, cud = (x.to(dev) for x in (q, k, v, beta, cu))
    s0d = None if S0 is None else S0.to(dev)
    H, T = w.H, q.shape[1]
    dt = _lib.EFLA_BF16 if w.dtype == "bf16" else _lib.EFLA_F32
    o = torch.empty((H, T, w.d_v), dtype=q.dtype, device=dev)
    S_L = torch.empty((n_seq, H, w.d_k, w.d_v), dtype=torch.float32, device=dev)
    need = _lib.efla_forward_varlen_workspace_size(n_seq, H, T, w.d_k, w.d_v, w.chunk, dt,
                                                   _lib.EFLA_PATH_AUTO)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    p = lambda x: None if x is None else x.data_ptr()  # noqa: E731

    def step():
        st = _lib.efla_forward_varlen_ex(p(qd), p(kd), p(vd), p(bd), p(cud), p(s0d), p(o),
                                         p(S_L), n_seq, H, T, w.d_k, w.d_v, w.chunk, dt,
                                         _lib.EFLA_EXACT, _lib.EFLA_PATH_AUTO, p(ws), need, sp)
        if st:
            raise RuntimeError(f"varlen forward failed: {_lib.status_string(st)}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    path = "fused" if need == 0 else ("segmented" if need > _lib.efla_forward_varlen_workspace_size(
        n_seq, H, T, w.d_k, w.d_v, w.chunk, dt, _lib.EFLA_PATH_STAGED) else "staged")
    return {"workload": name, "dtype": w.dtype, "path": path, "sequences": n_seq, "heads": H,
            "tokens_per_head": T, "longest": max(lengths), "shortest": min(lengths),
            "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
            "note": f"{name} recipe; random lengths; region of {args.steps} calls"}


def bench_config(args, name, dev):
    """Another workload, timed like the headline one on the path AUTO takes
    for it, with its roofline (fp32 workloads against the fp32 MFMA peak),
    warm and cold per-call times, and the fp64 oracle on the host beside it."""
    a = argparse.Namespace(**vars(args))
    a.path, a.no_compare = "auto", True
    w = wl.FORWARD_WORKLOADS[name]
    res, host = bench_forward(a, w, dev)
    out = {k: res[k] for k in ("ms_per_step", "tflops", "mfma_frac", "kernel_ms", "roofline",
                               "call_ms", "flops_per_token_head")}
    out["workload"] = w.name
    out["config"] = res["config"]
    out["dtype"] = w.dtype
    out["value"] = res["value"]
    out["unit"] = "tokens/s"
    out["token_heads_per_s"] = w.B * w.H * w.L / (res["ms_per_step"] * 1e-3)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, host)
    if w.recipe == "stiff":
        out["stiff_exact_vs_euler"] = stiff_compare(w, host, dev)
    return out


def stiff_compare(w, host, dev):
    """The stiff workload under both updates on the same kernels: the exact
    flow's state stays bounded, the explicit Euler step's (transition
    eigenvalue 1 - beta lambda, far below -1) overflows.  Kernel time of each
    and the size of the resulting state."""
    q, k, v, beta, S0 = host
    qd, kd, vd, bd = (x.to(dev) for x in (q, k, v, beta))
    s0d = None if S0 is None else S0.to(dev)
    res = {}
    for upd in ("exact", "euler"):
        efla.forward(qd, kd, vd, bd, s0d, chunk=w.chunk, update=upd)   # warm
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        o, S_L = efla.forward(qd, kd, vd, bd, s0d, chunk=w.chunk, update=upd)
        e1.record()
        torch.cuda.synchronize()
        fin = torch.isfinite(S_L)
        res[upd] = {"ms": e0.elapsed_time(e1),
                    "S_L_nonfinite_fraction": float((~fin).float().mean()),
                    "S_L_max_abs_finite": float(S_L[fin].abs().max()) if bool(fin.any()) else None}
    return res


def backward_flops_per_token(dk, dv, C):
    """The chunked backward as built, per token-head, including the forward
    recompute it needs (masked halves of C x C products not counted):
    state scan with stored states (W S, K^T E: 4 dk dv); UT transform
    (3 C dk + C dv + C^2/3); reverse scan (K dS, Q^T dO, W^T dE: 6 dk dv,
    A^T dO: C dv); gradient kernel (K S, dX S^T, E dS_out^T, dO S^T: 8 dk dv;
    Gamma, dA K, dA^T Q, dGam K, dGam^T K: 5 C dk; N D X, N^T dE, dE (DX)^T,
    dO E^T: 4 C dv; N, N^T dN, Z N^T: C^2)."""
    return 18 * dk * dv + 8 * C * dk + 6 * C * dv + 4 * C * C / 3.0 + 2 * dk


def grad_kernel_work(w, esz):
    """(flops, bytes) per launch of the per-chunk gradient kernel."""
    B, H, L, dk, dv, C = w.B, w.H, w.L, w.d_k, w.d_v, w.chunk
    n = B * H * L
    nch = B * H * ((L + C - 1) // C)
    flops = (8 * dk * dv + 5 * C * dk + 4 * C * dv + C * C) * n
    # reads q, k, v, dO; alpha, lambda, beta; each chunk's entry state, dS_out
    # and dE (stored in the input dtype); writes dq, dk, dv, dbeta
    byts = (n * (2 * dk + 2 * dv) * esz + 12 * n + 2 * nch * dk * dv * esz + nch * C * dv * esz +
            n * (2 * dk + dv) * esz + 4 * n)
    return flops, byts


def bench_backward(args, w, dev):
    """One backward pass (dq, dk, dv, dbeta, dS0) of the workload, given dO
    and dS_L; inputs, upstream gradients, outputs and workspace resident."""
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=0)
    dO, dSL = wl.output_grads(w, seed=0)
    qd, kd, vd, bd, s0d, dod, dsld = (None if x is None else x.to(dev)
                                      for x in (q, k, v, beta, S0, dO, dSL))
    dt = _lib.EFLA_BF16 if w.dtype == "bf16" else _lib.EFLA_F32
    B, H, L, dk, dv, C = w.B, w.H, w.L, w.d_k, w.d_v, w.chunk
    outs = [torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd),
            torch.empty_like(bd), torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)]
    need = _lib.efla_backward_workspace_size(B, H, L, dk, dv, C, dt)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    p = lambda x: None if x is None else x.data_ptr()  # noqa: E731

    def step():
        st = _lib.efla_backward(p(qd), p(kd), p(vd), p(bd), p(s0d), p(dod), p(dsld),
                                *[p(o) for o in outs], B, H, L, dk, dv, C, dt, _lib.EFLA_EXACT,
                                p(ws), need, sp)
        if st:
            raise RuntimeError(f"backward failed: {_lib.status_string(st)}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    n = B * H * L
    fl = backward_flops_per_token(dk, dv, C) * n
    gf, gb = grad_kernel_work(w, 2 if w.dtype == "bf16" else 4)
    return {"workload": w.name, "ms_per_step": ms, "tokens_per_s": B * L / (ms * 1e-3),
            "tflops": fl / (ms * 1e-3) / 1e12, "flops_per_token_head": fl / n,
            "workspace_bytes": need,
            "grad_kernel_algorithmic_flops": gf, "grad_kernel_algorithmic_bytes": gb,
            "note": "three launches: the UT transform (which also forms alpha and lambda), "
                    "the state scan storing chunk "
                    "entry states and the reverse state scan sharing one launch, per-chunk "
                    "gradients (bf16 MFMA for bf16 inputs, fp32 for the triangular chain); "
                    "per-kernel times from rocprofv3"}


def cpu_baseline(w, host, min_seconds=1.0):
    """The fp64 oracle on the host cores, timed on whole passes over the
    workload, repeated until min_seconds of wall time have elapsed (on 16
    threads about 16-30 s of CPU work).  It runs OpenMP over the B*H
    independent sequences, so the threads it can use are min(available
    threads, B*H); that is `cores`."""
    import oracle
    q, k, v, beta, S0 = host
    threads = oracle.max_threads()
    heads = w.B * w.H
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(q, k, v, beta, S0)
        passes += 1
        t = time.perf_counter() - t0
        if t >= min_seconds:
            break
    return {"value": passes * w.B * w.L / t, "unit": "tokens/s", "cores": min(threads, heads),
            "threads_available": threads, "cpu_model": cpu_model(),
            "kind": "oracle", "seconds": t, "passes": passes,
            "sample": f"{passes} whole pass(es) over the {w.name} workload ({heads} heads x "
                      f"{w.L} tokens), fp64, OpenMP over heads; inputs converted to fp64 "
                      f"before timing"}


def measured_peaks(dev):
    """What this GPU reaches in practice, beside the published peaks, from the
    library's own reference kernels (include/efla_peaks.h): a streaming copy
    of 1 GiB (bytes read + written per second) and loops of independent MFMAs
    on register operands, bf16 (v_mfma_f32_16x16x32_bf16) and fp32
    (v_mfma_f32_16x16x4_f32), eight workgroups of four waves per CU."""
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def time_ms(fn, n):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def check(st):
        if st:
            raise RuntimeError(f"peak kernel failed: {_lib.status_string(st)}")

    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t_copy = time_ms(lambda: check(_lib.efla_peak_copy(src.data_ptr(), dst.data_ptr(),
                                                       COPY_BYTES, sp)), 10)
    del src, dst
    out = {"hbm_copy_GB_s": 2 * COPY_BYTES / (t_copy * 1e-3) / 1e9}
    blocks = 256 * 8
    sink = torch.empty(blocks * 4, dtype=torch.float32, device=dev)
    for name, dt, iters in (("bf16", _lib.EFLA_BF16, 4000), ("f32", _lib.EFLA_F32, 2000)):
        fl = [0.0]

        def run():
            st, fl[0] = _lib.efla_peak_mfma(sink.data_ptr(), blocks, iters, dt, sp)
            check(st)
        t = time_ms(run, 5)
        out[f"{name}_mfma_TFLOP_s"] = fl[0] / (t * 1e-3) / 1e12
    out["note"] = ("library reference kernels: 1 GiB streaming copy (16-byte loads, "
                   "non-temporal stores); independent-MFMA loops on register operands, "
                   f"{blocks} workgroups x 4 waves; published peaks: 8 TB/s, 2.5 PFLOP/s bf16, "
                   "157.3 TFLOP/s fp32")
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# --- HBM traffic from rocprofv3 --pmc ----------------------------------------

COPY_BYTES = 1 << 30


def copy_calibration(args, dev):
    """A plain device copy of COPY_BYTES (read once, written once): the
    FETCH_SIZE / WRITE_SIZE it reads under rocprofv3 --pmc calibrate those
    counters to bytes.  Only torch's copy kernel runs (the source is left
    uninitialised so no fill kernel is launched)."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(max(args.steps, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": max(args.steps, 1)}), flush=True)


def _pmc_per_dispatch(csv_path, name_re, counter):
    """Average over matching dispatches of the counter summed over its
    dimensions (KiB for FETCH_SIZE / WRITE_SIZE)."""
    import csv
    per = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter or not re.search(name_re, row["Kernel_Name"]):
                continue
            d = int(row["Dispatch_Id"])
            per[d] = per.get(d, 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for /{name_re}/ in {csv_path}")
    return sum(per.values()) / len(per), len(per)


def pmc_summary(args):
    """Writes profiles/traffic_<kernel>_<workload>.txt from four rocprofv3
    --pmc runs under args.pmc_summary: fetch/ and write/ (this bench, one
    counter each) and cal_fetch/ and cal_write/ (--copy-calibration)."""
    import glob
    d = args.pmc_summary
    w = wl.FORWARD_WORKLOADS[args.workload]
    kname, kre, src = {"fused": ("fused", r"fused_kernel", "fused_forward.hip"),
                       "scan": ("scan", r"scan_kernel", "chunk_scan.hip"),
                       "ut": ("ut", r"ut_kernel", "ut_transform.hip"),
                       "decode": ("decode", r"decode_kernel", "coef_decode.hip")}[args.pmc_kernel]

    def csv_of(sub):
        hits = glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)
        if len(hits) != 1:
            raise SystemExit(f"expected one counter_collection.csv under {d}/{sub}, got {hits}")
        return hits[0]
    fk, nf = _pmc_per_dispatch(csv_of("fetch"), kre, "FETCH_SIZE")
    wk, nw = _pmc_per_dispatch(csv_of("write"), kre, "WRITE_SIZE")
    cfk, _ = _pmc_per_dispatch(csv_of("cal_fetch"), r"elementwise|copy", "FETCH_SIZE")
    cwk, _ = _pmc_per_dispatch(csv_of("cal_write"), r"elementwise|copy", "WRITE_SIZE")
    f_fac = COPY_BYTES / (cfk * 1024.0)
    w_fac = COPY_BYTES / (cwk * 1024.0)
    hbm = fk * 1024.0 * f_fac + wk * 1024.0 * w_fac
    esz = 2 if w.dtype == "bf16" else 4
    if kname == "decode":
        dw = wl.DECODE_WORKLOADS["decode-f32"]
        n = args.decode_only or 512
        algo = n * dw.H * (2 * dw.d_k * dw.d_v * 4 + (2 * dw.d_k + 2 * dw.d_v) * 4 + 4)
        wname = f"decode-f32-N{n}"
        bench_cmd = f"python bench.py --decode-only {n}"
    else:
        algo = (fused_work(w, esz, True)[1] if kname == "fused"
                else stage_work(w, esz)[kname][1])
        wname = w.name
        bench_cmd = (f"python bench.py --workload {w.name} --steps 5 --warmup 2 --no-decode "
                     "--no-cpu-baseline --no-backward --no-configs --no-peaks --no-cold")
    out = os.path.join(PROFILES, f"traffic_{kname}_{wname}.txt")
    lines = [
        f"HBM traffic of {kre} on {wname} from rocprofv3 --pmc (one counter per run)",
        f"  fetch: rocprofv3 --pmc FETCH_SIZE --kernel-include-regex {kre} --output-format csv -- {bench_cmd}",
        f"  write: rocprofv3 --pmc WRITE_SIZE --kernel-include-regex {kre} --output-format csv -- {bench_cmd}",
        "  calibration: the same two counters over python bench.py --copy-calibration --steps 5",
        f"source_sha256_16: {source_hash(src)}",
        f"fetch_kib_per_dispatch: {fk:.1f}  (mean of {nf} dispatches)",
        f"write_kib_per_dispatch: {wk:.1f}  (mean of {nw} dispatches)",
        f"copy_of_{COPY_BYTES}_bytes: FETCH_SIZE {cfk:.1f} KiB, WRITE_SIZE {cwk:.1f} KiB",
        f"fetch_factor: {f_fac:.4f}  write_factor: {w_fac:.4f}  (bytes per counted byte)",
        f"hbm_bytes_per_launch: {hbm:.6e}",
        f"algorithmic_bytes_per_launch: {algo:.6e}",
        f"traffic_over_algorithmic: {hbm / algo:.3f}",
    ]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed calls first; the GPU clocks take some tens of ms of load to settle")
    ap.add_argument("--workload", default="lm1.3b-bf16", choices=sorted(wl.FORWARD_WORKLOADS))
    ap.add_argument("--path", default="auto", choices=["auto", "staged", "fused", "segmented"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache per-call timing")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured copy / MFMA peaks")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the lm340m-bf16 and long-stiff-f32 forward lines")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip timing the Euler variant of the fused kernel")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (traffic counter calibration)")
    ap.add_argument("--pmc-summary", metavar="DIR",
                    help="write profiles/traffic_<kernel>_<workload>.txt from --pmc runs in DIR")
    ap.add_argument("--pmc-kernel", default="fused", choices=["fused", "scan", "ut", "decode"])
    ap.add_argument("--decode-only", type=int, metavar="N",
                    help="only time the decode step with N sequences (for --pmc runs)")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the operator shards over sequences/heads with no communication; run one "
              "process per GPU instead)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no HIP device visible", file=sys.stderr)
        sys.exit(1)
    _lib.lib()   # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(args, dev)
        return
    if args.decode_only:
        print(json.dumps(bench_decode(args, dev, n_seq=args.decode_only)), flush=True)
        return
    w = wl.FORWARD_WORKLOADS[args.workload]
    print(f"[bench] forward {w.name} path={args.path}", file=sys.stderr, flush=True)
    res, host = bench_forward(args, w, dev)
    if not args.no_decode:
        print("[bench] decode-f32", file=sys.stderr, flush=True)
        res["decode"] = bench_decode(args, dev)
        print("[bench] decode-f32 at N=512 (state twice the Infinity Cache)", file=sys.stderr,
              flush=True)
        res["decode_512"] = bench_decode(args, dev, n_seq=512)
    if not args.no_compare and w.dtype == "bf16":
        print("[bench] varlen", file=sys.stderr, flush=True)
        res["varlen"] = bench_varlen(args, dev)
        print("[bench] varlen long-stiff-f32", file=sys.stderr, flush=True)
        res["varlen_f32"] = bench_varlen(args, dev, "long-stiff-f32", n_seq=4)
    if not args.no_backward:
        print(f"[bench] backward {w.name}", file=sys.stderr, flush=True)
        res["backward"] = bench_backward(args, w, dev)
    if not args.no_configs:
        res["configs"] = {}
        for name in ("lm340m-bf16", "long-stiff-f32"):
            if name == w.name:
                continue
            print(f"[bench] forward {name}", file=sys.stderr, flush=True)
            res["configs"][name] = bench_config(args, name, dev)
    if not args.no_peaks:
        print("[bench] measured peaks", file=sys.stderr, flush=True)
        pk = measured_peaks(dev)
        # the HBM figure: the better of the reference copy and the decode step
        # at N = 512 (a state twice the Infinity Cache), which streams HBM too
        hbm = pk["hbm_copy_GB_s"]
        src = "reference copy kernel"
        if "decode_512" in res and res["decode_512"]["GB_s"] > hbm:
            hbm, src = res["decode_512"]["GB_s"], "decode step at N=512"
        pk["hbm_GB_s"], pk["hbm_source"] = hbm, src
        res["measured_peaks"] = pk

        def attach(rf, dtype):
            ref = hbm if rf["bound"] == "hbm" else pk[f"{dtype}_mfma_TFLOP_s"]
            rf["measured_peak"] = ref
            rf["frac_of_measured_peak"] = rf["achieved"] / ref
        attach(res["roofline"], w.dtype)
        for c in res.get("configs", {}).values():
            attach(c["roofline"], c["dtype"])
        if "decode" in res:
            for key in ("decode", "decode_512"):
                res[key]["frac_of_measured_hbm"] = res[key]["GB_s"] / hbm
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, host)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
