"""CPU: the Python binding rejects tensors that do not match what the C ABI sizes them
by, before anything reaches the library.

The library derives every extent from q's shape and dereferences every pointer on the
GPU, so an undersized out / lse / gradient tensor, a host tensor or a tensor on another
device would be read or written out of bounds. These checks run without a GPU: shape
and dtype mismatches are found first, then host tensors are refused.
"""

import ctypes

import pytest
import torch

from exact_attention_35_amd import capi


def _qkv(B=1, H=2, N=10, d=64, dv=64, dtype=torch.bfloat16):
    q = torch.zeros(B, H, N, d, dtype=dtype)
    k = torch.zeros(B, H, N, d, dtype=dtype)
    v = torch.zeros(B, H, N, dv, dtype=dtype)
    return q, k, v


def _status(exc):
    return exc.value.status


def test_out_and_lse_shapes_and_dtypes_are_checked():
    q, k, v = _qkv()
    with pytest.raises(capi.FaError) as e:
        capi.fa_fwd(q, k, v, out=torch.zeros(1, 2, 9, 64, dtype=torch.bfloat16))
    assert _status(e) == capi.STATUS["FA_ERR_SHAPE"]
    with pytest.raises(capi.FaError) as e:
        capi.fa_fwd(q, k, v, out=torch.zeros(1, 2, 10, 64, dtype=torch.float32))
    assert _status(e) == capi.STATUS["FA_ERR_DTYPE"]
    with pytest.raises(capi.FaError) as e:
        capi.fa_fwd(q, k, v, lse=torch.zeros(1, 2, 5))
    assert _status(e) == capi.STATUS["FA_ERR_SHAPE"]
    with pytest.raises(capi.FaError) as e:
        capi.fa_fwd(q, k, v, lse=torch.zeros(1, 2, 10, dtype=torch.float64))
    assert _status(e) == capi.STATUS["FA_ERR_DTYPE"]


def test_bias_must_broadcast():
    q, k, v = _qkv()
    with pytest.raises(capi.FaError) as e:
        capi.fa_fwd(q, k, v, bias=torch.zeros(1, 3, 10, 10))
    assert _status(e) == capi.STATUS["FA_ERR_SHAPE"]
    with pytest.raises(capi.FaError) as e:
        capi.fa_fwd(q, k, v, bias=torch.zeros(1, 2, 10, 9))
    assert _status(e) == capi.STATUS["FA_ERR_SHAPE"]


def test_host_tensors_are_refused_before_any_launch():
    q, k, v = _qkv()
    with pytest.raises(capi.FaError, match="not a device tensor"):
        capi.fa_fwd(q, k, v)
    with pytest.raises(capi.FaError, match="not a device tensor"):
        capi.fa_fwd_qk(q, k, v, causal=True)
    with pytest.raises(capi.FaError, match="not a device tensor"):
        capi.fa_fwd_ex(q, k, v, None)


def test_workspace_must_be_uint8():
    q, k, v = _qkv()
    with pytest.raises(capi.FaError) as e:
        capi.fa_fwd_ex(q, k, v, torch.zeros(16, dtype=torch.float32))
    assert _status(e) in (capi.STATUS["FA_ERR_WORKSPACE"], capi.STATUS["FA_ERR_NULL"])


def test_gradient_arguments_are_checked():
    q, k, v = _qkv()
    out = torch.zeros(1, 2, 10, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 10)
    do = torch.zeros(1, 2, 10, 64, dtype=torch.bfloat16)
    with pytest.raises(capi.FaError) as e:  # lse is required
        capi.fa_bwd(q, k, v, out, None, do)
    assert _status(e) == capi.STATUS["FA_ERR_NULL"]
    with pytest.raises(capi.FaError) as e:
        capi.fa_bwd(q, k, v, out, lse, do[:, :, :9])
    assert _status(e) == capi.STATUS["FA_ERR_SHAPE"]
    with pytest.raises(capi.FaError) as e:
        capi.fa_bwd(q, k, v, out, lse, do, grad_q=torch.zeros(1, 2, 10, 32, dtype=torch.bfloat16))
    assert _status(e) == capi.STATUS["FA_ERR_SHAPE"]
    with pytest.raises(capi.FaError) as e:
        capi.fa_bwd(q, k, v, out, lse, do, grad_v=torch.zeros(1, 2, 10, 64, dtype=torch.float16))
    assert _status(e) == capi.STATUS["FA_ERR_DTYPE"]
    with pytest.raises(capi.FaError, match="not a device tensor"):
        capi.fa_bwd(q, k, v, out, lse, do)


def test_launch_timer_arguments_are_checked():
    # out-of-range counts are refused by the binding and by the library itself, before any
    # event is created; arming zero launches and reading zero back touches no device
    for n in (-1, capi.FA_PROBE_TIMER_MAX + 1):
        with pytest.raises(capi.FaError):
            capi.fa_probe_timer_arm(n)
        assert capi.lib().fa_probe_timer_arm(n) == capi.STATUS["FA_ERR_NULL"]
    assert capi.lib().fa_probe_timer_read(None, 0) == capi.STATUS["FA_ERR_NULL"]
    capi.fa_probe_timer_arm(0)
    assert capi.fa_probe_timer_read(0) == []
    with pytest.raises(capi.FaError):
        capi.fa_probe_timer_read(1)      # nothing was armed and launched


def test_issue_probe_arguments_are_checked():
    # refused before any launch: null buffers, roles outside 0..4, unsupported op counts
    L = capi.lib()
    assert L.fa_probe_issue(0, 0, 0, 1, 1, None, None, None) == capi.STATUS["FA_ERR_NULL"]
    buf = ctypes.c_void_p(16)  # never dereferenced: every call below fails its checks first
    assert L.fa_probe_issue(5, 0, 0, 1, 1, buf, buf, None) == capi.STATUS["FA_ERR_NULL"]
    assert L.fa_probe_issue(-1, 0, 0, 1, 1, buf, buf, None) == capi.STATUS["FA_ERR_NULL"]
    assert L.fa_probe_issue(0, 0, 0, 0, 1, buf, buf, None) == capi.STATUS["FA_ERR_NULL"]
    assert L.fa_probe_issue(0, 3, 0, 1, 1, buf, buf, None) == capi.STATUS["FA_ERR_SHAPE"]
    assert L.fa_probe_issue(1, 4, 0, 1, 1, buf, buf, None) == capi.STATUS["FA_ERR_SHAPE"]


def test_read_probe_arguments_are_checked():
    L = capi.lib()
    buf = ctypes.c_void_p(16)
    assert L.fa_probe_read(None, 16, buf, 1, None) == capi.STATUS["FA_ERR_NULL"]
    assert L.fa_probe_read(buf, 16, None, 1, None) == capi.STATUS["FA_ERR_NULL"]
    assert L.fa_probe_read(buf, 24, buf, 1, None) == capi.STATUS["FA_ERR_NULL"]   # not a multiple of 16
    assert L.fa_probe_read(ctypes.c_void_p(8), 16, buf, 1, None) == capi.STATUS["FA_ERR_NULL"]  # misaligned


def test_lds_probe_arguments_are_checked():
    # refused before any launch: null buffers, empty grids or loops, unknown access kinds
    L = capi.lib()
    buf = ctypes.c_void_p(16)  # never dereferenced: every call below fails its checks first
    assert L.fa_probe_lds(0, 1, 1, None, buf, None) == capi.STATUS["FA_ERR_NULL"]
    assert L.fa_probe_lds(0, 1, 1, buf, None, None) == capi.STATUS["FA_ERR_NULL"]
    assert L.fa_probe_lds(0, 0, 1, buf, buf, None) == capi.STATUS["FA_ERR_NULL"]
    assert L.fa_probe_lds(0, 1, 0, buf, buf, None) == capi.STATUS["FA_ERR_NULL"]
    assert L.fa_probe_lds(5, 1, 1, buf, buf, None) == capi.STATUS["FA_ERR_SHAPE"]
    assert L.fa_probe_lds(-1, 1, 1, buf, buf, None) == capi.STATUS["FA_ERR_SHAPE"]


def test_tile_probe_arguments_are_checked():
    L = capi.lib()
    buf = ctypes.c_void_p(256)  # never dereferenced: every call below fails its checks first
    big = 1 << 18
    assert L.fa_probe_tile(0, 117, 1, 1, None, 0, None, buf, None) == capi.STATUS["FA_ERR_NULL"]
    assert L.fa_probe_tile(0, 117, 1, 0, None, 0, buf, buf, None) == capi.STATUS["FA_ERR_NULL"]
    assert L.fa_probe_tile(1, 117, 1, 1, None, big, buf, buf, None) == capi.STATUS["FA_ERR_NULL"]   # copies need src
    assert L.fa_probe_tile(1, 117, 1, 1, buf, big - 16, buf, buf, None) == capi.STATUS["FA_ERR_SHAPE"]  # too small
    assert L.fa_probe_tile(1, 117, 1, 1, ctypes.c_void_p(264), big, buf, buf, None) == capi.STATUS["FA_ERR_SHAPE"]
    assert L.fa_probe_tile(2, 117, 1, 1, buf, big, buf, buf, None) == capi.STATUS["FA_ERR_SHAPE"]
    assert L.fa_probe_tile(0, 100, 1, 1, None, 0, buf, buf, None) == capi.STATUS["FA_ERR_SHAPE"]
