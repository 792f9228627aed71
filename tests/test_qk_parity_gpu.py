"""GPU parity of fa_fwd_qk: N_q query rows against N_k keys (decoding steps included),
through the C ABI, against the fp64 oracle on the same seeded inputs.

The causal mask aligns the query rows to the end of the keys (key j allowed for row i
iff j <= i + N_k - N_q); rows that see no key (N_q > N_k) must come back as O = 0,
lse = -inf.
"""

import numpy as np
import pytest

from exact_attention_35_amd import capi, workloads
from oracle import sdpa_reference, sdpa_reference_rows
from parity_util import check_lse, check_out, to_np

pytestmark = pytest.mark.gpu


def _inputs(w, dev):
    inp = workloads.make_inputs(w, device="cpu")
    return inp, {n: (None if t is None else t.to(dev)) for n, t in inp.items()}


CASES = [  # (N_q, N_k, causal, bias, d, dv, B, H)
    (1, 1000, True, False, 128, 128, 2, 3),
    (1, 4097, True, False, 128, 128, 1, 4),
    (7, 1000, True, False, 64, 128, 1, 2),
    (200, 1000, True, False, 128, 64, 1, 2),
    (333, 777, False, True, 64, 64, 2, 2),
    (777, 333, True, False, 128, 128, 1, 2),   # more rows than keys: the first 444 see none
    (130, 130, True, False, 128, 128, 1, 1),
    (5, 64, True, True, 128, 128, 1, 3),
    (300, 0, False, False, 128, 128, 1, 1),    # no keys at all
    (3, 2000, True, False, 128, 128, 4, 40),   # 160 heads of one query tile: wide b*h split
    (40, 900, True, True, 64, 64, 2, 50),      # a short single tile: merge only its row groups
    # key ranges longer than the unit table's 9-bit fields (counted in granules of 2^s tiles)
    (1, 40000, True, False, 128, 128, 1, 1),
    (2, 65536, False, False, 64, 128, 1, 2),
    (130, 70000, True, False, 128, 128, 1, 1),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=[f"nq{c[0]}-nk{c[1]}-c{int(c[2])}-b{int(c[3])}-d{c[4]}-{c[5]}" for c in CASES])
def test_rectangular_elementwise(gpu_device, case, dtype):
    import torch

    nq, nk, causal, bias, d, dv, B, H = case
    w = workloads.workload(3).resized(B=B, H=H, N=nk, Nq=nq, d=d, dv=dv, causal=causal, bias=bias,
                                      dtype=dtype, seed=7000 + nq + nk)
    print(f"\n[qk] {case} {dtype}", flush=True)
    inp, gpu = _inputs(w, gpu_device)
    out = torch.full((B, H, nq, dv), float("nan"), dtype=gpu["q"].dtype, device=gpu_device)
    lse = torch.full((B, H, nq), float("nan"), dtype=torch.float32, device=gpu_device)
    capi.fa_fwd_qk(gpu["q"], gpu["k"], gpu["v"], bias=gpu["bias"], causal=causal, out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref, sc = sdpa_reference(inp["q"], inp["k"], inp["v"], inp["bias"], causal, allow_empty_rows=True,
                                      with_scale=True)
    check_out(out, o_ref, dtype, str(case), scale=sc)
    check_lse(lse, l_ref, str(case))


def test_square_problem_is_fa_fwd_bitwise(gpu_device):
    import torch

    w = workloads.workload(1).resized(N=1000)
    _, gpu = _inputs(w, gpu_device)
    a = capi.fa_fwd(gpu["q"], gpu["k"], gpu["v"], causal=True)
    b = capi.fa_fwd_qk(gpu["q"], gpu["k"], gpu["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_workload_full_size_sampled(gpu_device):
    # the benchmarked decoding step (one row per head against 8192 cached keys), in the
    # launch configuration the benchmark times, on sampled heads
    import torch

    w = workloads.WORKLOADS["bf16_decode_b8_h32_nk8192_d128"]
    inp, gpu = _inputs(w, gpu_device)
    out, lse = capi.fa_fwd_qk(gpu["q"], gpu["k"], gpu["v"], causal=True)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (3, 17), (7, 31)]:
        o_ref, l_ref, sc = sdpa_reference_rows(inp["q"], inp["k"], inp["v"], None, True, b, h, [0],
                                               with_scale=True)
        check_out(to_np(out[b, h, [0]]), o_ref, "bf16", f"decode b={b} h={h}", scale=sc)
        check_lse(to_np(lse[b, h, [0]]), l_ref, f"decode b={b} h={h}")


def test_decode_workspace_entry_matches(gpu_device):
    import torch

    w = workloads.workload(1).resized(B=2, H=4, N=3000, Nq=3)
    _, gpu = _inputs(w, gpu_device)
    a = capi.fa_fwd_qk(gpu["q"], gpu["k"], gpu["v"], causal=True)
    nbytes = capi.fa_fwd_qk_workspace_size(2, 4, 3, 3000, 128, 128, capi.FA_BF16, True)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=gpu_device)
    b = capi.fa_fwd_qk_ex(gpu["q"], gpu["k"], gpu["v"], ws, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_graph_capture_replays_match_eager(gpu_device):
    """A decoding step (one query row per head, split over keys) captured into a HIP graph
    gives bitwise the eager output on every replay."""
    import torch

    w = workloads.workload(1).resized(B=2, H=8, N=3000, Nq=1)
    _, gpu = _inputs(w, gpu_device)
    q, k, v = (gpu[n].clone() for n in ("q", "k", "v"))
    nbytes = capi.fa_fwd_qk_workspace_size(w.B, w.H, 1, w.N, w.d, w.dv, capi.FA_BF16, True)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=gpu_device)
    out = torch.empty(w.B, w.H, 1, w.dv, dtype=q.dtype, device=gpu_device)
    lse = torch.empty(w.B, w.H, 1, dtype=torch.float32, device=gpu_device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        capi.fa_fwd_qk_ex(q, k, v, ws, causal=True, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        capi.fa_fwd_qk_ex(q, k, v, ws, causal=True, out=out, lse=lse)
    gen = torch.Generator().manual_seed(13)
    for _ in range(3):
        q.copy_(torch.randn(q.shape, generator=gen).to(q.dtype).to(gpu_device))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_ref, l_ref = capi.fa_fwd_qk(q, k, v, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(lse, l_ref)
