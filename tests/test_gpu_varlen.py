"""Parity of efla_forward_varlen (packed sequences of varying length) with the
fp64 oracle run on each sequence alone, plus its structural properties."""
import pytest
import torch

import delta_rule_sequence_alpha_amd as efla
import efla_workloads as wl
import oracle
from tests._parity import TOL, dev, note, rel_err

pytestmark = pytest.mark.gpu


def _check_each(w, lengths, q, k, v, beta, cu, S0, o, S_L, update="exact"):
    eo = es = 0.0
    c = cu.tolist()
    for n, ln in enumerate(lengths):
        t0, t1 = c[n], c[n + 1]
        sl = lambda x: x[:, t0:t1][None]  # noqa: E731  [1, H, len, d]
        s0 = None if S0 is None else S0[n][None]
        o_r, S_r = oracle.forward(sl(q), sl(k), sl(v), beta[:, t0:t1][None], s0, update=update)
        if ln:
            eo = max(eo, rel_err(o[:, t0:t1][None], o_r))
        es = max(es, rel_err(S_L[n][None], S_r))
    print(f"  err o={eo:.3e} S_L={es:.3e}", flush=True)
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


@pytest.mark.parametrize("dk,dv,chunk,lengths", [
    (128, 128, 64, [0, 1, 15, 64, 65, 200, 127, 0, 300]),
    (64, 32, 32, [33, 0, 96, 7, 150]),
    (16, 128, 16, [5, 16, 17, 40]),
])
@pytest.mark.parametrize("with_s0", [True, False])
def test_varlen_parity(dk, dv, chunk, lengths, with_s0):
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(H=2, d_k=dk, d_v=dv, chunk=chunk)
    note(f"varlen dk={dk} dv={dv} C={chunk} lengths={lengths} S0={with_s0}")
    q, k, v, beta, cu, S0 = wl.varlen_inputs(w, lengths, seed=len(lengths))
    if not with_s0:
        S0 = None
    o, S_L = efla.forward_varlen(*dev(q, k, v, beta, cu), dev(S0) if S0 is not None else None,
                                 chunk=chunk)
    torch.cuda.synchronize()
    _check_each(w, lengths, q, k, v, beta, cu, S0, o, S_L)


def test_varlen_equal_lengths_match_fixed_length_bitwise():
    """Equal lengths: the same chunks and arithmetic as the fixed-length call."""
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(B=3, H=2, L=150)
    note("varlen vs fixed length")
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=21)
    o_f, S_f = efla.forward(*dev(q, k, v, beta, S0), chunk=64)
    # [B, H, L, d] -> [H, B*L, d]
    pk = lambda x: x.transpose(0, 1).reshape(w.H, w.B * w.L, *x.shape[3:]).contiguous()  # noqa: E731
    cu = torch.arange(0, w.B * w.L + 1, w.L, dtype=torch.int32)
    o_v, S_v = efla.forward_varlen(*dev(pk(q), pk(k), pk(v), pk(beta), cu, S0), chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(pk(o_f), o_v)
    assert torch.equal(S_f, S_v)


def test_varlen_leaves_tokens_outside_sequences_and_euler():
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(H=2)
    lengths = [40, 0, 90]
    note("varlen untouched tail + euler")
    q, k, v, beta, cu, S0 = wl.varlen_inputs(w, lengths, seed=5)
    T = q.shape[1]
    extra = 37   # tokens past the last sequence
    pad = lambda x: torch.cat([x, x[:, :extra]], dim=1)  # noqa: E731
    qd, kd, vd, bd = dev(pad(q), pad(k), pad(v), pad(beta))
    out = torch.full((2, T + extra, w.d_v), 7.0, dtype=torch.bfloat16, device="cuda")
    o, S_L = efla.forward_varlen(qd, kd, vd, bd, dev(cu), dev(S0), chunk=64, out=out,
                                 update="euler")
    torch.cuda.synchronize()
    assert torch.all(o[:, T:] == 7.0)
    _check_each(w, lengths, q, k, v, beta, cu, S0, o[:, :T], S_L, update="euler")


def test_varlen_many_sequences_sampled():
    """A large packed batch (64 sequences x 16 heads, 65536 tokens per head),
    checked on a sample of sequences."""
    w = wl.FORWARD_WORKLOADS["lm1.3b-bf16"].with_(H=16)
    lengths = wl.varlen_lengths(64, 65536, seed=3)
    note("varlen 64 sequences x 16 heads")
    q, k, v, beta, cu, S0 = wl.varlen_inputs(w, lengths, seed=3)
    o, S_L = efla.forward_varlen(*dev(q, k, v, beta, cu, S0), chunk=64)
    torch.cuda.synchronize()
    c = cu.tolist()
    for n in (0, 17, 63):
        t0, t1 = c[n], c[n + 1]
        for h in (0, 9):
            o_r, S_r = oracle.forward(q[h:h + 1, t0:t1][None], k[h:h + 1, t0:t1][None],
                                      v[h:h + 1, t0:t1][None], beta[h:h + 1, t0:t1][None],
                                      S0[n, h][None, None])
            if t1 > t0:
                assert rel_err(o[h:h + 1, t0:t1][None], o_r) <= TOL["bf16"]
            assert rel_err(S_L[n, h][None, None], S_r) <= TOL["bf16"]
