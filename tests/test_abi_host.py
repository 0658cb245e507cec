"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments before any HIP
call (every call below fails validation, so nothing touches a device)."""
import ctypes
import os
import re
import subprocess

import pytest

from delta_rule_sequence_alpha_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

FAKE = 0x10000        # a 16-byte-aligned pointer value that is never dereferenced
MISALIGNED = 0x10008


def header_functions():
    """Every function declared in include/*.h."""
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(efla_[a-z_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail(f"{_lib.LIB_PATH} not built (python -m delta_rule_sequence_alpha_amd.build)")
    return _lib.lib()


def test_library_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert len(declared) == 24
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (efla_[a-z_]+)\b", out))
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)
    assert sorted(n for n, _, _ in _lib.SIGNATURES) == declared


def test_status_strings(lib):
    names = ["EFLA_OK", "EFLA_ERR_INVALID_ARG", "EFLA_ERR_UNSUPPORTED", "EFLA_ERR_WORKSPACE",
             "EFLA_ERR_HIP"]
    for i, n in enumerate(names):
        assert _lib.status_string(i) == n
    assert _lib.status_string(77) == "EFLA_ERR_UNKNOWN"


def test_workspace_size(lib):
    # staged path: W + U (dtype) + A (dtype), each 256-byte aligned (the UT
    # transform forms alpha itself)
    B, H, L, d, C = 4, 16, 4096, 128, 64
    n = B * H * L
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    want = up(n * d * 2) + up(n * d * 2) + up(B * H * (L // C) * C * C * 2)
    assert _lib.efla_forward_workspace_size_ex(B, H, L, d, d, C, _lib.EFLA_BF16,
                                               _lib.EFLA_PATH_STAGED) == want
    assert _lib.efla_forward_workspace_size(1, 1, 64, 48, 16, 16, _lib.EFLA_F32) == 0  # unsupported
    assert _lib.efla_forward_workspace_size(1, 1, -1, 16, 16, 16, _lib.EFLA_F32) == 0  # invalid
    # ragged L rounds the chunk count up
    assert _lib.efla_forward_workspace_size_ex(1, 1, 65, 16, 16, 64, _lib.EFLA_F32,
                                               _lib.EFLA_PATH_STAGED) == \
        up(65 * 16 * 4) * 2 + up(2 * 64 * 64 * 4)


def _fwd(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, S0=None, o=FAKE, S_L=FAKE, B=1, H=1, L=64, dk=16,
             dv=16, chunk=16, dt=_lib.EFLA_F32, ws=FAKE, ws_bytes=1 << 30, path=0, stream=None)
    a.update(over)
    return _lib.efla_forward_ex(a["q"], a["k"], a["v"], a["beta"], a["S0"], a["o"], a["S_L"],
                                a["B"], a["H"], a["L"], a["dk"], a["dv"], a["chunk"], a["dt"],
                                a["ws"], a["ws_bytes"], a["path"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(dt=7), _lib.EFLA_ERR_INVALID_ARG),
    (dict(B=-1), _lib.EFLA_ERR_INVALID_ARG),
    (dict(L=-5), _lib.EFLA_ERR_INVALID_ARG),
    (dict(dk=0), _lib.EFLA_ERR_INVALID_ARG),
    (dict(chunk=-16), _lib.EFLA_ERR_INVALID_ARG),
    (dict(dk=48), _lib.EFLA_ERR_UNSUPPORTED),
    (dict(dv=256), _lib.EFLA_ERR_UNSUPPORTED),
    (dict(chunk=128), _lib.EFLA_ERR_UNSUPPORTED),
    (dict(q=None), _lib.EFLA_ERR_INVALID_ARG),
    (dict(beta=None), _lib.EFLA_ERR_INVALID_ARG),
    (dict(S_L=None), _lib.EFLA_ERR_INVALID_ARG),
    (dict(o=MISALIGNED), _lib.EFLA_ERR_INVALID_ARG),
    (dict(S0=MISALIGNED), _lib.EFLA_ERR_INVALID_ARG),
    (dict(ws=None), _lib.EFLA_ERR_WORKSPACE),
    (dict(ws_bytes=100), _lib.EFLA_ERR_WORKSPACE),
    (dict(ws=FAKE + 16), _lib.EFLA_ERR_INVALID_ARG),
    (dict(path=9), _lib.EFLA_ERR_INVALID_ARG),
])
def test_forward_validation(lib, over, status):
    assert _fwd(lib, **over) == status


def test_empty_batch_is_a_no_op(lib):
    # B*H == 0: nothing to do, no pointer is needed and nothing is launched
    assert _fwd(lib, B=0, q=None, k=None, v=None, beta=None, o=None, S_L=None, ws=None) == _lib.EFLA_OK


def test_decode_validation(lib):
    d = lambda **o: _lib.efla_decode_step(  # noqa: E731
        o.get("q", FAKE), FAKE, FAKE, FAKE, o.get("S", FAKE), FAKE, o.get("N", 2), 3,
        o.get("dk", 128), 128, o.get("dt", _lib.EFLA_F32), None)
    assert d(dt=3) == _lib.EFLA_ERR_INVALID_ARG
    assert d(N=-1) == _lib.EFLA_ERR_INVALID_ARG
    assert d(dk=100) == _lib.EFLA_ERR_UNSUPPORTED
    assert d(q=None) == _lib.EFLA_ERR_INVALID_ARG
    assert d(S=MISALIGNED) == _lib.EFLA_ERR_INVALID_ARG
    assert d(N=0) == _lib.EFLA_OK


def test_stage_validation(lib):
    assert _lib.efla_coefficients(FAKE, FAKE, FAKE, None, -1, 128, 0, None) == _lib.EFLA_ERR_INVALID_ARG
    assert _lib.efla_coefficients(FAKE, FAKE, FAKE, None, 10, 24, 0, None) == _lib.EFLA_ERR_UNSUPPORTED
    assert _lib.efla_coefficients(None, FAKE, FAKE, None, 10, 128, 0, None) == _lib.EFLA_ERR_INVALID_ARG
    assert _lib.efla_ut_transform(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 16, 16, 16, 0,
                                  None) == _lib.EFLA_ERR_INVALID_ARG
    assert _lib.efla_ut_transform(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 16, 16, 8, 0,
                                  None) == _lib.EFLA_ERR_UNSUPPORTED
    assert _lib.efla_chunk_scan(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 1, 1, 64, 16, 16,
                                16, 0, None) == _lib.EFLA_ERR_INVALID_ARG
    assert _lib.efla_chunk_scan(FAKE, FAKE, FAKE, FAKE, MISALIGNED, None, FAKE, FAKE, 1, 1, 64, 16,
                                16, 16, 0, None) == _lib.EFLA_ERR_INVALID_ARG


def test_update_variant_validation(lib):
    """The *_update entry points reject an unknown update before any HIP call,
    and otherwise validate exactly like the exact-update entry points."""
    def f(update, S_L=FAKE, dk=16):
        return _lib.efla_forward_update(FAKE, FAKE, FAKE, FAKE, None, FAKE, S_L, 1, 2, 64, dk, 16,
                                        16, _lib.EFLA_F32, FAKE, 1 << 30, 0, update, None)
    assert f(2) == _lib.EFLA_ERR_INVALID_ARG
    assert f(_lib.EFLA_EULER, S_L=None) == _lib.EFLA_ERR_INVALID_ARG
    assert f(_lib.EFLA_EULER, dk=24) == _lib.EFLA_ERR_UNSUPPORTED
    assert _lib.efla_decode_step_update(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 128, 128, 0, -1,
                                        None) == _lib.EFLA_ERR_INVALID_ARG
    assert _lib.efla_decode_step_update(FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 2, 128, 128, 0,
                                        _lib.EFLA_EULER, None) == _lib.EFLA_ERR_INVALID_ARG
    assert _lib.efla_coefficients_update(FAKE, FAKE, FAKE, None, 10, 128, 0, 7,
                                         None) == _lib.EFLA_ERR_INVALID_ARG
    assert _lib.efla_coefficients_update(FAKE, FAKE, FAKE, None, 10, 24, 0, _lib.EFLA_EULER,
                                         None) == _lib.EFLA_ERR_UNSUPPORTED


def test_varlen_validation(lib):
    def f(**o):
        a = dict(q=FAKE, cu=FAKE, S_L=FAKE, N=3, H=2, T=100, dk=64, dv=64, chunk=64,
                 dt=_lib.EFLA_BF16, update=0)
        a.update(o)
        return _lib.efla_forward_varlen(a["q"], FAKE, FAKE, FAKE, a["cu"], None, FAKE, a["S_L"],
                                        a["N"], a["H"], a["T"], a["dk"], a["dv"], a["chunk"],
                                        a["dt"], a["update"], None)
    assert f(dt=_lib.EFLA_F32) == _lib.EFLA_ERR_UNSUPPORTED   # fused path only
    assert f(N=-1) == _lib.EFLA_ERR_INVALID_ARG
    assert f(T=-1) == _lib.EFLA_ERR_INVALID_ARG
    assert f(dk=24) == _lib.EFLA_ERR_UNSUPPORTED
    assert f(update=5) == _lib.EFLA_ERR_INVALID_ARG
    assert f(cu=None) == _lib.EFLA_ERR_INVALID_ARG
    assert f(S_L=MISALIGNED) == _lib.EFLA_ERR_INVALID_ARG
    assert f(q=None) == _lib.EFLA_ERR_INVALID_ARG
    assert f(N=0, cu=None) == _lib.EFLA_OK     # nothing to do


def _varlen_ex(**o):
    a = dict(q=FAKE, cu=FAKE, S_L=FAKE, N=3, H=2, T=1000, dk=64, dv=64, chunk=64,
             dt=_lib.EFLA_F32, update=0, path=_lib.EFLA_PATH_STAGED, ws=FAKE, ws_bytes=1 << 30)
    a.update(o)
    return _lib.efla_forward_varlen_ex(a["q"], FAKE, FAKE, FAKE, a["cu"], None, FAKE, a["S_L"],
                                       a["N"], a["H"], a["T"], a["dk"], a["dv"], a["chunk"],
                                       a["dt"], a["update"], a["path"], a["ws"], a["ws_bytes"],
                                       None)


def test_varlen_ex_validation(lib):
    f = _varlen_ex
    need = _lib.efla_forward_varlen_workspace_size(3, 2, 1000, 64, 64, 64, _lib.EFLA_F32,
                                                   _lib.EFLA_PATH_STAGED)
    assert f(ws=None) == _lib.EFLA_ERR_WORKSPACE
    assert f(ws_bytes=need - 1) == _lib.EFLA_ERR_WORKSPACE
    assert f(ws=MISALIGNED) == _lib.EFLA_ERR_INVALID_ARG
    assert f(path=9) == _lib.EFLA_ERR_INVALID_ARG
    assert f(path=_lib.EFLA_PATH_FUSED) == _lib.EFLA_ERR_UNSUPPORTED   # no fp32 fused kernel
    assert f(N=-1) == _lib.EFLA_ERR_INVALID_ARG
    assert f(dk=24) == _lib.EFLA_ERR_UNSUPPORTED
    assert f(update=5) == _lib.EFLA_ERR_INVALID_ARG
    assert f(cu=None) == _lib.EFLA_ERR_INVALID_ARG
    assert f(S_L=MISALIGNED) == _lib.EFLA_ERR_INVALID_ARG
    assert f(q=None) == _lib.EFLA_ERR_INVALID_ARG
    assert f(N=0, cu=None, ws=None) == _lib.EFLA_OK    # nothing to do
    # grid bound: H * (ceil(T / C) + N) workgroups must fit an int
    assert f(N=1 << 24, H=64, T=1 << 20) == _lib.EFLA_ERR_UNSUPPORTED


def test_varlen_workspace_size(lib):
    # W, U, A by token (dtype) over H*T tokens, chunk offsets int32 [N+1]
    N, H, T, dk, dv, C = 5, 3, 1000, 64, 32, 32
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for dt, e in ((_lib.EFLA_F32, 4), (_lib.EFLA_BF16, 2)):
        want = up(H * T * dk * e) + up(H * T * dv * e) + up(H * T * C * e) + up((N + 1) * 4)
        assert _lib.efla_forward_varlen_workspace_size(N, H, T, dk, dv, C, dt,
                                                       _lib.EFLA_PATH_STAGED) == want
    assert _lib.efla_forward_varlen_workspace_size(N, H, T, dk, dv, C, _lib.EFLA_BF16,
                                                   _lib.EFLA_PATH_FUSED) == 0
    assert _lib.efla_forward_varlen_workspace_size(N, H, T, 24, dv, C, _lib.EFLA_F32,
                                                   _lib.EFLA_PATH_STAGED) == 0
    # few long sequences: AUTO takes the segmented scan (maps and entry states on top)
    seg = _lib.efla_forward_varlen_workspace_size(1, 16, 65536, 128, 128, 64, _lib.EFLA_F32,
                                                  _lib.EFLA_PATH_AUTO)
    stg = _lib.efla_forward_varlen_workspace_size(1, 16, 65536, 128, 128, 64, _lib.EFLA_F32,
                                                  _lib.EFLA_PATH_STAGED)
    assert seg > stg > 0
    # four packed fp32 sequences over 16 heads: too few scan workgroups, so segmented
    assert _lib.efla_forward_varlen_workspace_size(4, 16, 65536, 128, 128, 64, _lib.EFLA_F32,
                                                   _lib.EFLA_PATH_AUTO) == \
        _lib.efla_forward_varlen_workspace_size(4, 16, 65536, 128, 128, 64, _lib.EFLA_F32,
                                                _lib.EFLA_PATH_SEGMENTED) > \
        _lib.efla_forward_varlen_workspace_size(4, 16, 65536, 128, 128, 64, _lib.EFLA_F32,
                                                _lib.EFLA_PATH_STAGED)
    assert _lib.efla_forward_varlen_workspace_size(64, 16, 65536, 128, 128, 64, _lib.EFLA_F32,
                                                   _lib.EFLA_PATH_AUTO) == \
        _lib.efla_forward_varlen_workspace_size(64, 16, 65536, 128, 128, 64, _lib.EFLA_F32,
                                                _lib.EFLA_PATH_STAGED)


def test_auto_path_choice(lib):
    # bf16: the fused kernel, unless it would run <= 32 workgroups (sequences x
    # 32-column tiles) on sequences long enough to split; fp32: segmented scan
    # for few long sequences, else staged
    assert _lib.efla_forward_path(4, 16, 4096, 128, 128, 64, _lib.EFLA_BF16) == _lib.EFLA_PATH_FUSED
    assert _lib.efla_forward_path(1, 16, 65536, 128, 128, 64, _lib.EFLA_BF16) == _lib.EFLA_PATH_FUSED
    assert _lib.efla_forward_path(1, 8, 32768, 128, 128, 64, _lib.EFLA_BF16) == \
        _lib.EFLA_PATH_SEGMENTED
    assert _lib.efla_forward_path(1, 8, 256, 128, 128, 64, _lib.EFLA_BF16) == _lib.EFLA_PATH_FUSED
    assert _lib.efla_forward_workspace_size(1, 8, 32768, 128, 128, 64, _lib.EFLA_BF16) > 0
    assert _lib.efla_forward_varlen_workspace_size(2, 4, 32768, 128, 128, 64, _lib.EFLA_BF16,
                                                   _lib.EFLA_PATH_AUTO) > 0
    assert _lib.efla_forward_path(1, 16, 65536, 128, 128, 64, _lib.EFLA_F32) == _lib.EFLA_PATH_SEGMENTED
    assert _lib.efla_forward_path(1, 1, 64, 16, 16, 16, _lib.EFLA_F32) == _lib.EFLA_PATH_STAGED
    assert _lib.efla_forward_path(8, 16, 4096, 128, 128, 64, _lib.EFLA_F32) == _lib.EFLA_PATH_STAGED
    assert _lib.efla_forward_path(1, 1, 64, 24, 16, 16, _lib.EFLA_F32) == _lib.EFLA_PATH_AUTO
    seg = _lib.efla_forward_workspace_size_ex(1, 16, 65536, 128, 128, 64, _lib.EFLA_F32,
                                              _lib.EFLA_PATH_SEGMENTED)
    stg = _lib.efla_forward_workspace_size_ex(1, 16, 65536, 128, 128, 64, _lib.EFLA_F32,
                                              _lib.EFLA_PATH_STAGED)
    assert seg > stg > 0


def test_backward_workspace_size(lib):
    # alpha, lambda fp32; W, U, A, and per chunk the entry state, dS_out and dE (dtype)
    B, H, L, d, C = 4, 16, 4096, 128, 64
    n, nch = B * H * L, B * H * (L // C)
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    want = (2 * up(n * 4) + 2 * up(n * d * 2) + up(nch * C * C * 2) + 2 * up(nch * d * d * 2) +
            up(nch * C * d * 2))
    assert _lib.efla_backward_workspace_size(B, H, L, d, d, C, _lib.EFLA_BF16) == want
    assert _lib.efla_backward_workspace_size(1, 1, 0, 16, 16, 16, _lib.EFLA_F32) == 0
    assert _lib.efla_backward_workspace_size(1, 1, 64, 48, 16, 16, _lib.EFLA_F32) == 0


def _bwd(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, S0=None, d_o=FAKE, dS_L=None, dq=FAKE, dk_=FAKE,
             dv_=FAKE, dbeta=FAKE, dS0=FAKE, B=1, H=1, L=64, dk=16, dv=16, chunk=16,
             dt=_lib.EFLA_F32, update=_lib.EFLA_EXACT, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(over)
    return _lib.efla_backward(a["q"], a["k"], a["v"], a["beta"], a["S0"], a["d_o"], a["dS_L"],
                              a["dq"], a["dk_"], a["dv_"], a["dbeta"], a["dS0"], a["B"], a["H"],
                              a["L"], a["dk"], a["dv"], a["chunk"], a["dt"], a["update"], a["ws"],
                              a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(dt=7), _lib.EFLA_ERR_INVALID_ARG),
    (dict(update=2), _lib.EFLA_ERR_INVALID_ARG),
    (dict(L=-1), _lib.EFLA_ERR_INVALID_ARG),
    (dict(dk=48), _lib.EFLA_ERR_UNSUPPORTED),
    (dict(chunk=128), _lib.EFLA_ERR_UNSUPPORTED),
    (dict(d_o=None), _lib.EFLA_ERR_INVALID_ARG),
    (dict(dbeta=None), _lib.EFLA_ERR_INVALID_ARG),
    (dict(dq=MISALIGNED), _lib.EFLA_ERR_INVALID_ARG),
    (dict(dS_L=MISALIGNED), _lib.EFLA_ERR_INVALID_ARG),
    (dict(ws=None), _lib.EFLA_ERR_WORKSPACE),
    (dict(ws_bytes=100), _lib.EFLA_ERR_WORKSPACE),
    (dict(ws=FAKE + 16), _lib.EFLA_ERR_INVALID_ARG),
])
def test_backward_rejects_bad_arguments(lib, over, status):
    assert _bwd(lib, **over) == status


@pytest.mark.parametrize("cfg,status", [
    (dict(fused_scan_waves=3), _lib.EFLA_ERR_INVALID_ARG),
    (dict(scan_waves=3), _lib.EFLA_ERR_INVALID_ARG),
    (dict(bwd_scan_waves=8), _lib.EFLA_ERR_INVALID_ARG),
    (dict(scan_waves=8), _lib.EFLA_ERR_WORKSPACE),   # valid: fails on the workspace after
    (dict(scan_waves=-1), _lib.EFLA_ERR_INVALID_ARG),
    # valid values pass the check and validation goes on to the next error
    (dict(fused_scan_waves=1, scan_waves=4, bwd_scan_waves=2), _lib.EFLA_ERR_WORKSPACE),
    (None, _lib.EFLA_ERR_WORKSPACE),
])
def test_launch_config_validation(lib, cfg, status):
    """The launch configuration is an argument: out-of-range wave counts are
    rejected before any HIP call, on the forward and the backward entry."""
    assert _lib.efla_forward_config(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, 2, 64, 16, 16, 16,
                                    _lib.EFLA_F32, None, 0, _lib.EFLA_PATH_STAGED, _lib.EFLA_EXACT,
                                    cfg, None) == status
    assert _lib.efla_backward_config(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, 1, 2, 64, 16, 16, 16, _lib.EFLA_F32,
                                     _lib.EFLA_EXACT, cfg, None, 0, None) == status


def test_library_reads_no_environment():
    """No entry point depends on the process environment: the library imports
    no getenv/secure_getenv."""
    out = subprocess.run(["nm", "-D", "--undefined-only", _lib.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    assert not re.search(r"\b(secure_)?getenv\b", out)


def test_peak_kernel_validation(lib):
    """The peak reference kernels validate before any HIP call."""
    assert _lib.efla_peak_copy(None, FAKE, 1024, None) == _lib.EFLA_ERR_INVALID_ARG
    assert _lib.efla_peak_copy(FAKE, MISALIGNED, 1024, None) == _lib.EFLA_ERR_INVALID_ARG
    assert _lib.efla_peak_copy(FAKE, FAKE + 4096, 1000, None) == _lib.EFLA_ERR_INVALID_ARG  # not x16
    assert _lib.efla_peak_copy(FAKE, FAKE + 512, 1024, None) == _lib.EFLA_ERR_INVALID_ARG   # overlap
    assert _lib.efla_peak_copy(FAKE, FAKE + 4096, 0, None) == _lib.EFLA_OK                 # nothing
    assert _lib.efla_peak_mfma(None, 1, 1, _lib.EFLA_BF16, None)[0] == _lib.EFLA_ERR_INVALID_ARG
    assert _lib.efla_peak_mfma(FAKE, 0, 1, _lib.EFLA_BF16, None)[0] == _lib.EFLA_ERR_INVALID_ARG
    assert _lib.efla_peak_mfma(FAKE, 1, 0, _lib.EFLA_F32, None)[0] == _lib.EFLA_ERR_INVALID_ARG
    assert _lib.efla_peak_mfma(FAKE, 1, 1, 5, None)[0] == _lib.EFLA_ERR_INVALID_ARG


def test_noalloc_rejects_shapes_beyond_its_scratch(lib):
    """efla_forward_noalloc validates like efla_forward_update and refuses a
    staged or segmented shape whose intermediates exceed its fixed scratch,
    before any HIP call."""
    def f(**o):
        a = dict(B=1, H=2, L=64, dk=16, dv=16, chunk=16, dt=_lib.EFLA_F32, path=_lib.EFLA_PATH_STAGED,
                 update=_lib.EFLA_EXACT, q=FAKE, S_L=FAKE)
        a.update(o)
        return _lib.efla_forward_noalloc(a["q"], FAKE, FAKE, FAKE, None, FAKE, a["S_L"], a["B"],
                                         a["H"], a["L"], a["dk"], a["dv"], a["chunk"], a["dt"],
                                         a["path"], a["update"], None)
    big = dict(B=4, H=16, L=4096, dk=128, dv=128, chunk=64)     # 168 MB of intermediates (bf16)
    need = _lib.efla_forward_workspace_size_ex(4, 16, 4096, 128, 128, 64, _lib.EFLA_BF16,
                                               _lib.EFLA_PATH_STAGED)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert f(dt=_lib.EFLA_BF16, **big) == _lib.EFLA_ERR_WORKSPACE
    assert f(dt=_lib.EFLA_F32, path=_lib.EFLA_PATH_SEGMENTED, B=1, H=16, L=65536, dk=128, dv=128,
             chunk=64) == _lib.EFLA_ERR_WORKSPACE
    assert f(dt=7) == _lib.EFLA_ERR_INVALID_ARG
    assert f(update=3) == _lib.EFLA_ERR_INVALID_ARG
    assert f(path=9) == _lib.EFLA_ERR_INVALID_ARG
    assert f(dk=24) == _lib.EFLA_ERR_UNSUPPORTED
    assert f(S_L=None) == _lib.EFLA_ERR_INVALID_ARG
    assert f(q=MISALIGNED) == _lib.EFLA_ERR_INVALID_ARG
    assert f(B=0) == _lib.EFLA_OK          # nothing to do, nothing launched


def test_indexed_decode_validation(lib):
    """efla_decode_step_indexed validates before any HIP call; N = 0 is a
    no-op that needs no pointers."""
    def d(**o):
        a = dict(q=FAKE, slots=FAKE, S=FAKE, N=4, H=2, P=8, dk=128, dv=128, dt=_lib.EFLA_F32,
                 update=_lib.EFLA_EXACT)
        a.update(o)
        return _lib.efla_decode_step_indexed(a["q"], FAKE, FAKE, FAKE, a["slots"], a["S"], FAKE,
                                             None, a["N"], a["H"], a["P"], a["dk"], a["dv"],
                                             a["dt"], a["update"], None)
    assert d(dt=4) == _lib.EFLA_ERR_INVALID_ARG
    assert d(update=2) == _lib.EFLA_ERR_INVALID_ARG
    assert d(N=-1) == _lib.EFLA_ERR_INVALID_ARG
    assert d(P=-1) == _lib.EFLA_ERR_INVALID_ARG
    assert d(dk=48) == _lib.EFLA_ERR_UNSUPPORTED
    assert d(slots=None) == _lib.EFLA_ERR_INVALID_ARG
    assert d(S=None) == _lib.EFLA_ERR_INVALID_ARG
    assert d(S=MISALIGNED) == _lib.EFLA_ERR_INVALID_ARG
    assert d(q=None) == _lib.EFLA_ERR_INVALID_ARG
    assert d(N=0, q=None, slots=None, S=None) == _lib.EFLA_OK
