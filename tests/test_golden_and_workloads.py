"""The stored tiny-f32 oracle fixture, and the input generators' recipes."""
import os

import numpy as np
import pytest
import torch

import efla_workloads as wl
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_f32_oracle.txt")


def _read_golden():
    sections, cur = {}, None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line in ("o", "S_L"):
                cur = sections.setdefault(line, [])
                continue
            cur.append([float(x) for x in line.split()])
    return np.array(sections["o"]), np.array(sections["S_L"])


def test_oracle_reproduces_stored_tiny_fixture():
    w = wl.FORWARD_WORKLOADS["tiny-f32"]
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=0)
    o, SL = oracle.forward(q, k, v, beta, S0)
    go, gS = _read_golden()
    np.testing.assert_allclose(o.reshape(64, 16), go, rtol=0, atol=1e-14)
    np.testing.assert_allclose(SL.reshape(16, 16), gS, rtol=0, atol=1e-14)


def test_generator_is_seeded_and_shaped():
    w = wl.FORWARD_WORKLOADS["tiny-f32"]
    a = wl.forward_inputs(w, seed=0)
    b = wl.forward_inputs(w, seed=0)
    c = wl.forward_inputs(w, seed=1)
    for x, y in zip(a[:4], b[:4]):
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0])
    q, k, v, beta, S0 = a
    assert q.shape == (1, 1, 64, 16) and v.shape == (1, 1, 64, 16) and beta.shape == (1, 1, 64)
    assert S0 is None
    lam = (k.double() ** 2).sum(-1)
    assert lam.min() >= 0.01 * (1 - 1e-6) and lam.max() <= 16 * (1 + 1e-6)
    assert beta.min() >= 0 and beta.max() <= 1


@pytest.mark.parametrize("name", ["lm340m-bf16", "lm1.3b-bf16", "long-stiff-f32"])
def test_generator_recipes_at_reduced_length(name):
    w = wl.FORWARD_WORKLOADS[name].with_(L=256, B=1)
    q, k, v, beta, S0 = wl.forward_inputs(w, seed=0)
    assert q.dtype == (torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    assert k.shape == (1, w.H, 256, w.d_k) and v.shape == (1, w.H, 256, w.d_v)
    lam = (k.double() ** 2).sum(-1)
    if name == "lm340m-bf16":
        assert lam.min() > 0.2 and lam.max() < 4.2
        assert S0 is None
    elif name == "lm1.3b-bf16":
        assert 0.6 < lam.mean() < 1.4 and S0 is not None
        assert 0.015 < float(S0.std()) < 0.025
    else:
        assert lam.max() <= 1e4 * (1 + 1e-5) and lam.min() >= 0.01 * (1 - 1e-5)
        assert beta.max() <= 5
        # lambda > 100 only happens at a x10 spike (unspiked norms are at most 10)
        big = (lam > 100.0 * (1 + 1e-5))
        assert big.any()
        assert 0.005 < float(big.double().mean()) < 0.05


def test_decode_generator():
    w = wl.DECODE_WORKLOADS["decode-f32"]
    S = wl.decode_state(w, seed=0, n_seq=2)
    assert S.shape == (2, 16, 128, 128)
    q, k, v, beta = wl.decode_tokens(w, step=3, seed=0, n_seq=2)
    q2, _, _, _ = wl.decode_tokens(w, step=3, seed=0, n_seq=2)
    assert torch.equal(q, q2)
    assert q.shape == (2, 16, 128) and beta.shape == (2, 16)
    assert 0.04 < float(S.std()) < 0.06
