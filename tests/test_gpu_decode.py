"""Parity of efla_decode_step with the fp64 oracle (the recurrent form)."""
import numpy as np
import pytest
import torch

import delta_rule_sequence_alpha_amd as efla
import efla_workloads as wl
import oracle
from tests._parity import TOL, dev, note, rel_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (16, 128), (128, 16)])
def test_decode_shapes(dtype, dk, dv):
    w = wl.DecodeWorkload("d", 5, 3, dk, dv, 3, dtype)
    note(f"decode {dtype} dk={dk} dv={dv}")
    S = wl.decode_state(w, seed=1)
    Sd = dev(S)
    S_ref = S.double().numpy()
    for step in range(3):
        q, k, v, beta = wl.decode_tokens(w, step, seed=1)
        o = efla.decode_step(*dev(q, k, v, beta), Sd)
        torch.cuda.synchronize()
        o_r, S_ref = oracle.decode(q, k, v, beta, S_ref)
        assert rel_err(o, o_r) <= TOL[dtype]
        assert rel_err(Sd, S_ref) <= 1e-5   # the state itself is fp32 on both sides


def test_decode_degenerate_tokens():
    w = wl.DecodeWorkload("d", 2, 2, 64, 64, 1, "f32")
    note("decode degenerate tokens")
    S = wl.decode_state(w, seed=2)
    q, k, v, beta = wl.decode_tokens(w, 0, seed=2)
    k[0, 0] = 0.0
    beta[1, 1] = 0.0
    Sd = dev(S)
    o = efla.decode_step(*dev(q, k, v, beta), Sd)
    torch.cuda.synchronize()
    assert torch.equal(Sd[0, 0].cpu(), S[0, 0])
    assert torch.equal(Sd[1, 1].cpu(), S[1, 1])
    o_r, S_r = oracle.decode(q, k, v, beta, S)
    assert rel_err(o, o_r) <= 1e-5 and rel_err(Sd, S_r) <= 1e-5


def test_decode_steps_equal_forward():
    """L decode steps reproduce the chunked forward over the same tokens."""
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(B=2, H=2, L=70, dtype="f32")
    note("decode steps == forward")
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=8)
    qd, kd, vd, bd, sd = dev(q, k, v, beta, S0)
    o_f, S_f = efla.forward(qd, kd, vd, bd, sd, chunk=64)
    S = sd.clone()
    outs = []
    for t in range(w.L):
        outs.append(efla.decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                                     vd[:, :, t].contiguous(), bd[:, :, t].contiguous(), S))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, dim=2)
    assert rel_err(o_d, o_f.double().cpu().numpy()) <= 1e-4
    assert rel_err(S, S_f.double().cpu().numpy()) <= 1e-4


def test_decode_full_workload_1000_steps_sampled():
    """decode-f32 at full size (256 x 16 heads, d=128) for its 1000 steps; the
    oracle follows a fixed sample of 24 (n, h) heads through every step."""
    w = wl.DECODE_WORKLOADS["decode-f32"]
    note("decode-f32 full size, 1000 steps")
    rng = np.random.default_rng(0)
    sample_n = torch.from_numpy(rng.choice(w.N, size=24, replace=False))
    sample_h = torch.from_numpy(rng.integers(0, w.H, size=24))
    S = wl.decode_state(w, seed=0)
    S_ref = S[sample_n, sample_h].double().numpy()[:, None]      # [24,1,dk,dv]
    Sd = dev(S)
    del S
    worst_o = worst_s = 0.0
    for step in range(w.steps):
        q, k, v, beta = wl.decode_tokens(w, step, seed=0)
        o = efla.decode_step(*dev(q, k, v, beta), Sd)
        sel = (sample_n, sample_h)
        o_r, S_ref = oracle.decode(q[sel][:, None], k[sel][:, None], v[sel][:, None],
                                   beta[sel][:, None], S_ref)
        if step in (0, w.steps - 1) or step % 100 == 0:
            torch.cuda.synchronize()
            seld = (sample_n.cuda(), sample_h.cuda())
            eo = rel_err(o[seld][:, None], o_r)
            es = rel_err(Sd[seld][:, None], S_ref)
            worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
            print(f"  step {step}: err o={eo:.3e} S={es:.3e}", flush=True)
            assert eo <= TOL["f32"] and es <= TOL["f32"]
    print(f"  worst err o={worst_o:.3e} S={worst_s:.3e}", flush=True)
