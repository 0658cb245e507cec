"""The segmented state scan (path="segmented"): the sequence is split over L
into segments whose affine maps are formed in parallel, composed into entry
states, and replayed.  Parity with the fp64 oracle and with the plain staged
scan, at sizes where the split happens (at least 16 chunks per sequence)."""
import pytest
import torch

import delta_rule_sequence_alpha_amd as efla
import efla_workloads as wl
import oracle
from tests._parity import TOL, dev, note, rel_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,chunk,L,with_s0", [(128, 128, 64, 64 * 40 + 5, False),
                                                   (128, 128, 64, 64 * 33, True),
                                                   (64, 32, 32, 32 * 50 + 31, True),
                                                   (32, 64, 16, 16 * 70 + 3, False),
                                                   (16, 16, 16, 16 * 24, True)])
def test_segmented_parity(dtype, dk, dv, chunk, L, with_s0):
    w = wl.FORWARD_WORKLOADS["long-stiff-f32"].with_(B=1, H=3, L=L, d_k=dk, d_v=dv, chunk=chunk,
                                                     dtype=dtype)
    note(f"segmented {dtype} dk={dk} dv={dv} C={chunk} L={L} S0={with_s0}")
    q, k, v, beta, _ = wl.forward_inputs(w, seed=L)
    S0 = torch.randn(1, 3, dk, dv, generator=torch.Generator().manual_seed(L)) * 0.1 if with_s0 else None
    qd, kd, vd, bd = dev(q, k, v, beta)
    s0d = None if S0 is None else dev(S0)
    o, S_L = efla.forward(qd, kd, vd, bd, s0d, chunk=chunk, path="segmented")
    o_s, S_s = efla.forward(qd, kd, vd, bd, s0d, chunk=chunk, path="staged")
    torch.cuda.synchronize()
    o_r, S_r = oracle.forward(q, k, v, beta, S0)
    eo, es = rel_err(o, o_r), rel_err(S_L, S_r)
    print(f"  err o={eo:.3e} S_L={es:.3e}; vs staged o={rel_err(o, o_s.double().cpu().numpy()):.3e}",
          flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_segmented_is_auto_for_long_few_head_fp32_and_matches_full_size():
    """long-stiff-f32 at full size (16 heads x 65536 tokens) takes the
    segmented scan under AUTO; sampled heads against the oracle."""
    w = wl.FORWARD_WORKLOADS["long-stiff-f32"]
    note("segmented long-stiff-f32 full size (auto)")
    assert (efla.workspace_size(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, torch.float32, "auto")
            == efla.workspace_size(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, torch.float32, "segmented")
            > efla.workspace_size(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, torch.float32, "staged"))
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=0)
    o, S_L = efla.forward(*dev(q, k, v, beta), None, chunk=w.chunk)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S_L).all()
    for h in (0, 11):
        sl = (slice(0, 1), slice(h, h + 1))
        o_r, S_r = oracle.forward(q[sl], k[sl], v[sl], beta[sl], None)
        assert rel_err(o[sl], o_r) <= TOL["f32"] and rel_err(S_L[sl], S_r) <= TOL["f32"]


def test_segmented_euler():
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(B=1, H=2, L=64 * 32, dtype="f32")
    note("segmented euler")
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=9)
    o, S_L = efla.forward(*dev(q, k, v, beta, S0), chunk=64, path="segmented", update="euler")
    torch.cuda.synchronize()
    o_r, S_r = oracle.forward(q, k, v, beta, S0, update="euler")
    assert rel_err(o, o_r) <= TOL["f32"] and rel_err(S_L, S_r) <= TOL["f32"]
