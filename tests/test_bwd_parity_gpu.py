"""GPU parity of the gradients: fa_bwd (through the C ABI) against the fp64 gradient
oracle on the same seeded inputs.

The forward runs first (fa_fwd gives O and lse, as a training step would); the oracle
forms the gradients from Q, K, V and dO alone, by the definition. Small cases compare
every element; the full-size workloads compare sampled query rows (dQ) and key rows
(dK, dV), which the oracle computes one by one.
"""

import numpy as np
import pytest

from exact_attention_35_amd import capi, workloads
from oracle import sdpa_backward_reference, sdpa_backward_reference_sampled
from parity_util import check_grad, to_np

pytestmark = pytest.mark.gpu


def _device_inputs(w, dev):
    inp = workloads.make_inputs(w, device="cpu")
    inp["do"] = workloads.make_grad_out(w, device="cpu")
    gpu = {}
    for n, t in inp.items():
        if t is None:
            gpu[n] = None
        elif w.layout == "bnhd" and n in ("q", "k", "v", "do"):
            gpu[n] = t.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
        else:
            gpu[n] = t.to(dev)
    return inp, gpu


def _fwd_bwd(gpu, w):
    import torch

    out, lse = capi.fa_fwd(gpu["q"], gpu["k"], gpu["v"], bias=gpu["bias"], causal=w.causal)
    dq, dk, dv = capi.fa_bwd(gpu["q"], gpu["k"], gpu["v"], out, lse, gpu["do"], bias=gpu["bias"],
                             causal=w.causal)
    torch.cuda.synchronize()
    return dq, dk, dv


SMALL = [
    (1, dict(N=1000)),
    (1, dict(N=333, H=2)),
    (2, dict(B=2, H=4, N=777)),
    (3, dict(B=2, H=3, N=555)),
    (4, dict(H=2, N=1500)),
    (1, dict(N=700, causal=False)),
    (3, dict(B=2, H=64, N=300)),   # more b*h than a split plan takes: one unit per tile
    (2, dict(B=1, H=1, N=4000)),   # long single head: tiles cut into chunks
]


@pytest.mark.parametrize("idx,over", SMALL, ids=[f"w{i}-{o}" for i, o in SMALL])
def test_gradients_small_elementwise(gpu_device, idx, over):
    w = workloads.workload(idx).resized(**over)
    print(f"\n[bwd] {w.name} {over}", flush=True)
    inp, gpu = _device_inputs(w, gpu_device)
    dq, dk, dv = _fwd_bwd(gpu, w)
    rq, rk, rv, (sq, sk, sv) = sdpa_backward_reference(inp["q"], inp["k"], inp["v"], inp["do"], inp["bias"],
                                                       w.causal, with_scales=True)
    e = [check_grad(dq, rq, sq, "dQ"), check_grad(dk, rk, sk, "dK"), check_grad(dv, rv, sv, "dV")]
    print(f"[bwd] worst |err| / bound: dQ {e[0]:.3g} dK {e[1]:.3g} dV {e[2]:.3g}", flush=True)


# Split plans under other unit targets (FA_BWD_UNITS) cut the tiles into other chunk
# counts and lengths. Plans are cached per shape, so each case uses a shape that no other
# test plans, and the target is read when that shape is planned first.
UNIT_TARGETS = [(96, dict(N=2600)), (320, dict(N=2700)), (200, dict(H=2, N=2300, causal=False))]


@pytest.mark.parametrize("units,over", UNIT_TARGETS, ids=[f"u{u}-{o}" for u, o in UNIT_TARGETS])
def test_gradients_under_other_unit_targets(gpu_device, monkeypatch, units, over):
    monkeypatch.setenv("FA_BWD_UNITS", str(units))
    w = workloads.workload(1).resized(**over)
    print(f"\n[bwd] {w.name} {over} units={units}", flush=True)
    inp, gpu = _device_inputs(w, gpu_device)
    dq, dk, dv = _fwd_bwd(gpu, w)
    rq, rk, rv, (sq, sk, sv) = sdpa_backward_reference(inp["q"], inp["k"], inp["v"], inp["do"], inp["bias"],
                                                       w.causal, with_scales=True)
    check_grad(dq, rq, sq, "dQ")
    check_grad(dk, rk, sk, "dK")
    check_grad(dv, rv, sv, "dV")


@pytest.mark.parametrize("N", [1, 17, 65, 129, 255])
@pytest.mark.parametrize("d,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("causal,bias", [(True, False), (False, True)])
def test_gradients_odd_sizes(gpu_device, N, d, dv, causal, bias):
    w = workloads.workload(3).resized(B=1, H=2, N=N, d=d, dv=dv, causal=causal, bias=bias,
                                      seed=9000 + N)
    inp, gpu = _device_inputs(w, gpu_device)
    dq, dk, dv_ = _fwd_bwd(gpu, w)
    rq, rk, rv, (sq, sk, sv) = sdpa_backward_reference(inp["q"], inp["k"], inp["v"], inp["do"], inp["bias"],
                                                       causal, with_scales=True)
    check_grad(dq, rq, sq, f"dQ N={N}")
    check_grad(dk, rk, sk, f"dK N={N}")
    check_grad(dv_, rv, sv, f"dV N={N}")


def test_gradients_bitwise_reproducible_and_workspace_entry(gpu_device):
    import torch

    w = workloads.workload(1).resized(N=1100, H=2)
    _, gpu = _device_inputs(w, gpu_device)
    a = _fwd_bwd(gpu, w)
    b = _fwd_bwd(gpu, w)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    out, lse = capi.fa_fwd(gpu["q"], gpu["k"], gpu["v"], causal=True)
    nbytes = capi.fa_bwd_workspace_size(w.B, w.H, w.N, w.d, w.dv, capi.FA_BF16, True)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=gpu_device)
    c = capi.fa_bwd_ex(gpu["q"], gpu["k"], gpu["v"], out, lse, gpu["do"], ws, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, c):
        assert torch.equal(x, y)


FULL = [
    # (workload index, [(b, h)], sampled query rows, sampled key rows)
    (1, [(0, 0)], [0, 1, 127, 128, 4095, 8000, 8191], [0, 1, 63, 64, 4000, 8190, 8191]),
    (2, [(3, 31), (1, 7)], [0, 100, 2047, 4095], [0, 64, 3000, 4095]),
    (3, [(1, 15), (0, 2)], [0, 1, 1023, 2047], [0, 5, 1500, 2047]),
    (4, [(0, 3)], [0, 1, 127, 128, 16000, 32766, 32767], [0, 1, 63, 64, 20000, 32766, 32767]),
]


@pytest.mark.parametrize("idx,bhs,rows,keys", FULL, ids=[f"w{f[0]}" for f in FULL])
def test_gradients_full_size_sampled(gpu_device, idx, bhs, rows, keys):
    w = workloads.workload(idx)
    print(f"\n[bwd] full {w.name}", flush=True)
    inp, gpu = _device_inputs(w, gpu_device)
    dq, dk, dv = _fwd_bwd(gpu, w)
    for b, h in bhs:
        rq, rk, rv, (sq, sk, sv) = sdpa_backward_reference_sampled(
            inp["q"], inp["k"], inp["v"], inp["do"], inp["bias"], w.causal, b, h, rows, keys, with_scales=True)
        e = [check_grad(to_np(dq[b, h, rows]), rq, sq, f"dQ {w.name} b={b} h={h}"),
             check_grad(to_np(dk[b, h, keys]), rk, sk, f"dK {w.name} b={b} h={h}"),
             check_grad(to_np(dv[b, h, keys]), rv, sv, f"dV {w.name} b={b} h={h}")]
        print(f"[bwd] b={b} h={h} worst |err| / bound: dQ {e[0]:.3g} dK {e[1]:.3g} dV {e[2]:.3g}", flush=True)


def test_key_gradients_sum_to_zero(gpu_device):
    # rows of dS sum to zero, so the dK rows of every (b, h) add up to ~0
    w = workloads.workload(1).resized(N=2000, H=3)
    _, gpu = _device_inputs(w, gpu_device)
    _, dk, _ = _fwd_bwd(gpu, w)
    g = to_np(dk)
    tot = np.abs(g.sum(axis=2))
    scale = np.abs(g).sum(axis=2)
    assert (tot <= 2e-2 * scale + 1e-3).all()


F16 = [  # (workload index, overrides): the fp16 gradient kernels
    (1, dict(N=1000)),
    (3, dict(B=2, H=3, N=555)),
    (2, dict(B=2, H=4, N=777)),
]


@pytest.mark.parametrize("idx,over", F16, ids=[f"w{i}-{o}" for i, o in F16])
def test_fp16_gradients(gpu_device, idx, over):
    w = workloads.workload(idx).resized(dtype="f16", **over)
    inp, gpu = _device_inputs(w, gpu_device)
    dq, dk, dv = _fwd_bwd(gpu, w)
    rq, rk, rv, (sq, sk, sv) = sdpa_backward_reference(inp["q"], inp["k"], inp["v"], inp["do"], inp["bias"],
                                                       w.causal, with_scales=True)
    e = [check_grad(dq, rq, sq, "dQ", "f16"), check_grad(dk, rk, sk, "dK", "f16"),
         check_grad(dv, rv, sv, "dV", "f16")]
    print(f"[bwd f16] worst |err| / bound: dQ {e[0]:.3g} dK {e[1]:.3g} dV {e[2]:.3g}", flush=True)


def test_gradient_graph_capture_replays_match_eager(gpu_device):
    """fa_bwd_ex of a split problem (row statistics, gradient grid, chunk reduction)
    captured into a HIP graph gives, on every replay, bitwise the eager gradients for the
    inputs of that replay; eager work runs between the replays."""
    import torch

    w = workloads.workload(1).resized(N=1500)
    _, gpu = _device_inputs(w, gpu_device)
    q, k, v, g = (gpu[n].clone() for n in ("q", "k", "v", "do"))
    out, lse = capi.fa_fwd(q, k, v, causal=True)
    nbytes = capi.fa_bwd_workspace_size(w.B, w.H, w.N, w.d, w.dv, capi.FA_BF16, True)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=gpu_device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        capi.fa_bwd_ex(q, k, v, out, lse, g, ws, causal=True, grad_q=dq, grad_k=dk, grad_v=dv)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        capi.fa_bwd_ex(q, k, v, out, lse, g, ws, causal=True, grad_q=dq, grad_k=dk, grad_v=dv)
    gen = torch.Generator().manual_seed(12)
    for _ in range(3):
        g.copy_(torch.randn(g.shape, generator=gen).to(g.dtype).to(gpu_device))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = capi.fa_bwd(q, k, v, out, lse, g, causal=True)
        torch.cuda.synchronize()
        for x, y in zip((dq, dk, dv), ref):
            assert torch.equal(x, y)
