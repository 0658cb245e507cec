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


# --- slot-indexed decode over a state pool (ragged serving batches) ---------

def _pool(P, H, dk, dv, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(P, H, dk, dv, generator=g) * 0.05


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 32), (128, 128), (16, 16)])
def test_indexed_decode_updates_its_slots_only(dtype, dk, dv):
    """Token n updates pool entry slots[n] exactly as the recurrence does for
    that state (oracle on the gathered states); every other entry is left
    bit for bit as it was (Methodology 3, the recurrent form)."""
    P, H = 10, 3
    slots = [7, 2, 9, 0]
    w = wl.DecodeWorkload("d", len(slots), H, dk, dv, 1, dtype)
    note(f"indexed decode {dtype} dk={dk} dv={dv} slots={slots}")
    pool = _pool(P, H, dk, dv, seed=dk + dv)
    q, k, v, beta = wl.decode_tokens(w, 0, seed=3)
    pd = dev(pool)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = efla.decode_step_indexed(*dev(q, k, v, beta), torch.tensor(slots, dtype=torch.int32).cuda(),
                                 pd, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    o_r, S_r = oracle.decode(q, k, v, beta, pool[slots])
    assert rel_err(o, o_r) <= TOL[dtype]
    assert rel_err(pd[slots], S_r) <= 1e-5
    others = [i for i in range(P) if i not in slots]
    assert torch.equal(pd[others].cpu(), pool[others])


def test_indexed_decode_rejects_repeated_and_out_of_range_slots():
    """A slot named twice, or outside the pool, is rejected on the device:
    its tokens leave the pool untouched and output NaN, and err records why;
    the valid tokens of the same batch are applied."""
    P, H, d = 8, 2, 64
    slots = [3, 5, 3, 11, -1]
    w = wl.DecodeWorkload("d", len(slots), H, d, d, 1, "f32")
    note(f"indexed decode rejection slots={slots}")
    pool = _pool(P, H, d, d, seed=5)
    q, k, v, beta = wl.decode_tokens(w, 0, seed=5)
    pd = dev(pool)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = efla.decode_step_indexed(*dev(q, k, v, beta), torch.tensor(slots, dtype=torch.int32).cuda(),
                                 pd, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 3          # 1: repeated, 2: out of range
    oc = o.cpu()
    for n in (0, 2, 3, 4):
        assert torch.isnan(oc[n]).all()
    assert torch.isfinite(oc[1]).all()
    o_r, S_r = oracle.decode(q[1:2], k[1:2], v[1:2], beta[1:2], pool[5:6])
    assert rel_err(oc[1:2], o_r) <= 1e-5 and rel_err(pd[5:6], S_r) <= 1e-5
    untouched = [i for i in range(P) if i != 5]
    assert torch.equal(pd[untouched].cpu(), pool[untouched])


def test_indexed_decode_empty_batch_and_identity_slots():
    """N = 0 does nothing; slots = 0..N-1 on a pool of N is the plain decode
    step, bit for bit."""
    H, d = 2, 32
    pool = _pool(4, H, d, d, seed=6)
    pd = dev(pool)
    e = torch.empty(0, H, d, device="cuda")
    o = efla.decode_step_indexed(e, e, e, torch.empty(0, H, device="cuda"),
                                 torch.empty(0, dtype=torch.int32, device="cuda"), pd)
    torch.cuda.synchronize()
    assert o.shape == (0, H, d) and torch.equal(pd.cpu(), pool)
    w = wl.DecodeWorkload("d", 4, H, d, d, 1, "f32")
    q, k, v, beta = wl.decode_tokens(w, 0, seed=6)
    note("indexed decode identity slots")
    a, b = dev(pool), dev(pool)
    oa = efla.decode_step_indexed(*dev(q, k, v, beta), torch.arange(4, dtype=torch.int32).cuda(), a)
    ob = efla.decode_step(*dev(q, k, v, beta), b)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(a, b)


def test_indexed_decode_full_size_pool():
    """The decode workload's batch (256 sequences x 16 heads, d = 128) as a
    random subset of a 512-entry pool, checked on sampled sequences."""
    w = wl.DECODE_WORKLOADS["decode-f32"]
    P = 2 * w.N
    note(f"indexed decode full size N={w.N} P={P}")
    pool = wl.decode_state(dataclass_replace(w, N=P), seed=0)
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(0))[: w.N].to(torch.int32)
    q, k, v, beta = wl.decode_tokens(w, 0, seed=0)
    pd = dev(pool)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = efla.decode_step_indexed(*dev(q, k, v, beta), perm.cuda(), pd, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for n in (0, 77, 255):
        s = int(perm[n])
        o_r, S_r = oracle.decode(q[n:n + 1], k[n:n + 1], v[n:n + 1], beta[n:n + 1], pool[s:s + 1])
        assert rel_err(o[n:n + 1], o_r) <= TOL["f32"] and rel_err(pd[s:s + 1], S_r) <= TOL["f32"]
    unused = sorted(set(range(P)) - set(perm.tolist()))[:16]
    assert torch.equal(pd[unused].cpu(), pool[unused])


def dataclass_replace(w, **kw):
    import dataclasses
    return dataclasses.replace(w, **kw)
