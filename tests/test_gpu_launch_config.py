"""Parity of the kernel variants behind the launch configuration.

efla_forward_config and efla_backward_config take an explicit
efla_launch_config_t: fused_scan_waves (scan waves of the fused kernel: 2
runs 32-column tiles, 1 runs 16-column tiles), scan_waves (waves per
workgroup of the staged and segmented state scans; 8 exists for fp32 at
d_k = d_v = 128 and acts as 4 elsewhere) and bwd_scan_waves (the
backward's two scans).  Each value selects other compiled instances than the
defaults, so each is checked against the fp64 oracle here: a ragged bf16
forward on the fused and staged paths, an fp32 staged forward, a segmented
forward and a backward in both dtypes.
"""
import pytest
import torch

import delta_rule_sequence_alpha_amd as efla
import efla_workloads as wl
import oracle
from tests._parity import TOL, dev, note, rel_err

pytestmark = pytest.mark.gpu

OVERRIDES = [("fused_scan_waves", 1), ("fused_scan_waves", 2),
             ("scan_waves", 1), ("scan_waves", 2), ("scan_waves", 4), ("scan_waves", 8),
             ("bwd_scan_waves", 1), ("bwd_scan_waves", 2), ("bwd_scan_waves", 4)]


def _forward(w, path, seed, config):
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=seed)
    note(f"forward {w.name} {w.dtype} B={w.B} H={w.H} L={w.L} path={path} config={config}")
    o, S_L = efla.forward(*dev(q, k, v, beta, S0), chunk=w.chunk, path=path, config=config)
    torch.cuda.synchronize()
    o_r, S_r = oracle.forward(q, k, v, beta, S0)
    eo, es = rel_err(o, o_r), rel_err(S_L, S_r)
    print(f"  {path} {w.dtype}: err o={eo:.3e} S_L={es:.3e}", flush=True)
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


@pytest.mark.parametrize("field,value", OVERRIDES)
def test_forward_under_config(field, value):
    cfg = {field: value}
    bf = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(name="ovr", B=1, H=3, L=64 * 3 + 29)
    _forward(bf, "fused", seed=11, config=cfg)
    _forward(bf, "staged", seed=12, config=cfg)
    f32 = wl.FORWARD_WORKLOADS["long-stiff-f32"].with_(name="ovr", B=1, H=2, L=64 * 5 + 3)
    _forward(f32, "staged", seed=13, config=cfg)
    # few long sequences: the segment plan splits them (summary, combine, replay)
    seg = wl.FORWARD_WORKLOADS["long-stiff-f32"].with_(name="ovr", B=1, H=2, L=64 * 24 + 9)
    _forward(seg, "segmented", seed=14, config=cfg)


@pytest.mark.parametrize("field,value", OVERRIDES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_under_config(field, value, dtype):
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(name="ovr", B=1, H=2, L=64 * 2 + 21, dtype=dtype)
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=15)
    dO, dSL = wl.output_grads(w, seed=15)
    note(f"backward {dtype} L={w.L} {field}={value}")
    got = efla.backward(*dev(q, k, v, beta, S0, dO, dSL), chunk=w.chunk, config={field: value})
    torch.cuda.synchronize()
    ref = oracle.backward(q, k, v, beta, S0, dO, dSL)
    for name, g, r in zip(["dq", "dk", "dv", "dbeta", "dS0"], got, ref):
        e = rel_err(g, r)
        assert e <= TOL[dtype], (name, e)
