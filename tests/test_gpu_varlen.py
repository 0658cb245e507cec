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


# --- the staged and segmented paths (fp32 and bf16) ---------------------------

def _pad_tail(x, extra):
    """Append `extra` tokens past the last sequence (seeded |N(0, 1)| values,
    which the operator reads but must not use)."""
    g = torch.Generator().manual_seed(extra)
    t = torch.randn((x.shape[0], extra, *x.shape[2:]), generator=g).abs().to(x.dtype)
    return torch.cat([x, t], dim=1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["staged", "segmented"])
@pytest.mark.parametrize("dk,dv,chunk,lengths", [
    (128, 128, 64, [0, 1, 15, 64, 65, 200, 127, 0, 300]),
    (64, 32, 32, [33, 0, 96, 7, 150]),
    (16, 128, 16, [5, 16, 17, 40]),
    (32, 64, 64, [0, 0]),
])
def test_varlen_chunked_paths_parity(dtype, path, dk, dv, chunk, lengths):
    """Packed sequences on the UT transform + state scan kernels, each sequence
    against the oracle run on it alone.  A tail of tokens outside every
    sequence makes the token axis long enough for the segmented path to split
    each sequence (most segments of the short ones are empty), and must be
    left untouched."""
    w = wl.FORWARD_WORKLOADS["long-stiff-f32"].with_(H=2, d_k=dk, d_v=dv, chunk=chunk,
                                                     dtype=dtype)
    extra = 24 * chunk
    note(f"varlen {path} {dtype} dk={dk} dv={dv} C={chunk} lengths={lengths} tail={extra}")
    q, k, v, beta, cu, S0 = wl.varlen_inputs(w, lengths, seed=11 + len(lengths))
    T = q.shape[1]
    N, H = len(lengths), w.H
    ws = {p: efla.varlen_workspace_size(N, H, T + extra, dk, dv, chunk, q.dtype, path=p)
          for p in ("staged", "segmented")}
    if path == "segmented":   # the plan does split
        assert ws["segmented"] > ws["staged"] > 0
    qd, kd, vd, bd = dev(_pad_tail(q, extra), _pad_tail(k, extra), _pad_tail(v, extra),
                         _pad_tail(beta, extra))
    out = torch.full((H, T + extra, dv), 7.0, dtype=q.dtype, device="cuda")
    o, S_L = efla.forward_varlen(qd, kd, vd, bd, dev(cu), dev(S0), chunk=chunk, out=out,
                                 path=path)
    torch.cuda.synchronize()
    assert torch.all(o[:, T:] == 7.0)
    _check_each(w, lengths, q, k, v, beta, cu, S0, o[:, :T], S_L)


@pytest.mark.parametrize("path", ["staged", "segmented"])
def test_varlen_chunked_paths_euler_no_s0(path):
    w = wl.FORWARD_WORKLOADS["long-stiff-f32"].with_(H=3, d_k=64, d_v=64, chunk=32)
    lengths = [70, 0, 33, 400]
    note(f"varlen {path} f32 euler, no S0")
    q, k, v, beta, cu, _ = wl.varlen_inputs(w, lengths, seed=29)
    o, S_L = efla.forward_varlen(*dev(q, k, v, beta, cu), None, chunk=32, update="euler",
                                 path=path)
    torch.cuda.synchronize()
    _check_each(w, lengths, q, k, v, beta, cu, None, o, S_L, update="euler")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_varlen_staged_equal_lengths_match_fixed_length_bitwise(dtype):
    """Equal lengths on the staged path: the same chunks and arithmetic as the
    fixed-length staged call."""
    w = wl.FORWARD_WORKLOADS["long-stiff-f32"].with_(B=3, H=2, L=150, dtype=dtype)
    note(f"varlen staged {dtype} vs fixed length")
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=23)
    o_f, S_f = efla.forward(*dev(q, k, v, beta, S0), chunk=64, path="staged")
    pk = lambda x: x.transpose(0, 1).reshape(w.H, w.B * w.L, *x.shape[3:]).contiguous()  # noqa: E731
    cu = torch.arange(0, w.B * w.L + 1, w.L, dtype=torch.int32)
    o_v, S_v = efla.forward_varlen(*dev(pk(q), pk(k), pk(v), pk(beta), cu, S0), chunk=64,
                                   path="staged")
    torch.cuda.synchronize()
    assert torch.equal(pk(o_f), o_v)
    assert torch.equal(S_f, S_v)


def test_varlen_segmented_long_stiff_sampled():
    """The long-context fp32 case at full size: 65536 tokens per head in four
    sequences (one of them empty) over 16 heads, on the path AUTO picks
    (segmented), checked on sampled (sequence, head) pairs."""
    w = wl.FORWARD_WORKLOADS["long-stiff-f32"]
    lengths = [40000, 0, 9000, 16536]
    N, H, T = len(lengths), w.H, sum(lengths)
    seg = efla.varlen_workspace_size(N, H, T, 128, 128, 64, torch.float32, path="segmented")
    assert efla.varlen_workspace_size(N, H, T, 128, 128, 64, torch.float32) == seg > \
        efla.varlen_workspace_size(N, H, T, 128, 128, 64, torch.float32, path="staged")
    note("varlen long-stiff-f32 full size, auto path")
    q, k, v, beta, cu, S0 = wl.varlen_inputs(w, lengths, seed=31)
    o, S_L = efla.forward_varlen(*dev(q, k, v, beta, cu, S0), chunk=64)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S_L).all()
    c = cu.tolist()
    for n, h in ((0, 0), (2, 7), (3, 15), (1, 4)):
        t0, t1 = c[n], c[n + 1]
        o_r, S_r = oracle.forward(q[h:h + 1, t0:t1][None], k[h:h + 1, t0:t1][None],
                                  v[h:h + 1, t0:t1][None], beta[h:h + 1, t0:t1][None],
                                  None if S0 is None else S0[n, h][None, None])
        if t1 > t0:
            assert rel_err(o[h:h + 1, t0:t1][None], o_r) <= TOL["f32"]
        assert rel_err(S_L[n, h][None, None], S_r) <= TOL["f32"]


@pytest.mark.parametrize("path", ["staged", "segmented", "fused"])
def test_varlen_offsets_are_clamped(path):
    """Offsets outside [0, T] are clamped into it (the first below 0, the last
    past T): the sequences become [0, 40), [40, 40), [40, 90), [90, T), each
    equal to the oracle run on that range."""
    dtype = "bf16" if path == "fused" else "f32"
    w = wl.FORWARD_WORKLOADS["long-stiff-f32"].with_(H=2, d_k=64, d_v=64, chunk=32, dtype=dtype)
    lengths = [40, 0, 50, 130]
    note(f"varlen clamped offsets {path} {dtype}")
    q, k, v, beta, cu, S0 = wl.varlen_inputs(w, lengths, seed=37)
    T = q.shape[1]
    bad = torch.tensor([-7, 40, 40, 90, T + 1000], dtype=torch.int32)
    o, S_L = efla.forward_varlen(*dev(q, k, v, beta, bad), dev(S0) if S0 is not None else None,
                                 chunk=32, path=path)
    torch.cuda.synchronize()
    _check_each(w, lengths, q, k, v, beta, cu, S0, o, S_L)


@pytest.mark.parametrize("path", ["staged", "segmented", "fused"])
def test_varlen_many_short_sequences(path):
    """1000 packed sequences (many empty or shorter than a chunk) of one head
    pair: the chunk-offset prefix over a long offset array (staged and
    segmented, fp32), and the fused kernel past the sequence count it orders
    longest first (bf16), checked on a sample of sequences."""
    dtype = "bf16" if path == "fused" else "f32"
    w = wl.FORWARD_WORKLOADS["long-stiff-f32"].with_(H=2, d_k=32, d_v=32, chunk=16, dtype=dtype)
    lengths = wl.varlen_lengths(1000, 20000, seed=41)
    note(f"varlen 1000 sequences {dtype} {path}")
    q, k, v, beta, cu, S0 = wl.varlen_inputs(w, lengths, seed=41)
    o, S_L = efla.forward_varlen(*dev(q, k, v, beta, cu), None, chunk=16, path=path)
    torch.cuda.synchronize()
    c = cu.tolist()
    picks = [0, 1, 2, 499, 500, 998, 999] + [i for i, n in enumerate(lengths) if n == 0][:2] + \
        [max(range(1000), key=lambda i: lengths[i])]
    for n in picks:
        t0, t1 = c[n], c[n + 1]
        o_r, S_r = oracle.forward(q[:, t0:t1][None], k[:, t0:t1][None], v[:, t0:t1][None],
                                  beta[:, t0:t1][None], None)
        if t1 > t0:
            assert rel_err(o[:, t0:t1][None], o_r) <= TOL[dtype], n
        assert rel_err(S_L[n][None], S_r) <= TOL[dtype], n
