"""GPU: fa_fwd_qk_noalloc, the entry point that allocates no device memory (its split
partial states live in the library's fixed per-GPU scratch array), against fa_fwd_qk
through the C ABI on the same inputs.

Both run the same plan and kernels, so their outputs are compared bitwise, over two calls
in a row whose second is smaller (the array keeps the first call's contents), and the
results are also checked against the oracle.
"""

import numpy as np
import pytest

from exact_attention_35_amd import capi, workloads
from oracle import sdpa_reference
from parity_util import check_lse, check_out

pytestmark = pytest.mark.gpu


def _case(w, dev):
    import torch

    inp = workloads.make_inputs(w, device="cpu")
    g = {n: (None if t is None else t.to(dev)) for n, t in inp.items()}
    out = torch.full((w.B, w.H, w.n_q, w.dv), float("nan"), dtype=g["q"].dtype, device=dev)
    lse = torch.full((w.B, w.H, w.n_q), float("nan"), dtype=torch.float32, device=dev)
    return inp, g, out, lse


@pytest.mark.parametrize("first,second", [
    # (workload index, overrides): a larger split problem, then a smaller one
    ((1, dict(N=3000)), (1, dict(N=1000))),
    ((1, dict(B=2, H=8, N=4000, Nq=2)), (3, dict(B=1, H=2, N=700, Nq=300))),
    ((4, dict(H=2, N=2500)), (1, dict(N=200, Nq=50))),
])
def test_noalloc_matches_allocating_entry_point(gpu_device, first, second):
    import torch

    for idx, over in (first, second):
        w = workloads.workload(idx).resized(**over)
        print(f"\n[noalloc] {w.name} {over}", flush=True)
        inp, g, out, lse = _case(w, gpu_device)
        assert capi.fa_fwd_qk_workspace_size(w.B, w.H, w.n_q, w.N, w.d, w.dv, capi.FA_BF16, w.causal) > 0
        capi.fa_fwd_qk_noalloc(g["q"], g["k"], g["v"], out, lse, bias=g["bias"], causal=w.causal)
        ref_o, ref_l = capi.fa_fwd_qk(g["q"], g["k"], g["v"], bias=g["bias"], causal=w.causal)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        o_ref, l_ref, sc = sdpa_reference(inp["q"], inp["k"], inp["v"], inp["bias"], w.causal, with_scale=True)
        check_out(out, o_ref, "bf16", f"noalloc {over}", scale=sc)
        check_lse(lse, l_ref, f"noalloc {over}")


def test_noalloc_requires_outputs(gpu_device):
    w = workloads.workload(1).resized(N=300)
    _, g, out, lse = _case(w, gpu_device)
    with pytest.raises(capi.FaError):
        capi.fa_fwd_qk_noalloc(g["q"], g["k"], g["v"], None, lse, causal=True)
    # an unsplit problem (no scratch needed) goes through as well
    w2 = workloads.workload(2).resized(B=4, H=16, N=1024)
    inp2, g2, o2, l2 = _case(w2, gpu_device)
    assert capi.fa_fwd_qk_workspace_size(w2.B, w2.H, w2.N, w2.N, w2.d, w2.dv, capi.FA_BF16, True) == 0
    capi.fa_fwd_qk_noalloc(g2["q"], g2["k"], g2["v"], o2, l2, causal=True)
    ref = capi.fa_fwd_qk(g2["q"], g2["k"], g2["v"], causal=True)
    import torch

    torch.cuda.synchronize()
    assert torch.equal(o2, ref[0]) and torch.equal(l2, ref[1])
    assert np.isfinite(l2.cpu().numpy()).all()


def test_noalloc_fp16_then_bf16(gpu_device):
    """fp16 partial states in the same scratch array, then a bf16 call over them."""
    import torch

    w = workloads.workload(1).resized(N=2600)
    inp, g, _, _ = _case(w, gpu_device)
    h = {n: g[n].to(torch.float16) for n in ("q", "k", "v")}
    out = torch.full((w.B, w.H, w.N, w.dv), float("nan"), dtype=torch.float16, device=gpu_device)
    lse = torch.full((w.B, w.H, w.N), float("nan"), dtype=torch.float32, device=gpu_device)
    assert capi.fa_fwd_qk_workspace_size(w.B, w.H, w.N, w.N, w.d, w.dv, capi.FA_F16, True) > 0
    capi.fa_fwd_qk_noalloc(h["q"], h["k"], h["v"], out, lse, causal=True)
    ref_o, ref_l = capi.fa_fwd_qk(h["q"], h["k"], h["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    q16, k16, v16 = (h[n].cpu() for n in ("q", "k", "v"))
    o_ref, l_ref, sc = sdpa_reference(q16, k16, v16, None, True, with_scale=True)
    check_out(out, o_ref, "f16_mfma", "noalloc fp16", scale=sc)
    check_lse(lse, l_ref, "noalloc fp16")
    # a smaller bf16 call after it
    w2 = workloads.workload(1).resized(N=1500)
    inp2, g2, o2, l2 = _case(w2, gpu_device)
    capi.fa_fwd_qk_noalloc(g2["q"], g2["k"], g2["v"], o2, l2, causal=True)
    r2 = capi.fa_fwd_qk(g2["q"], g2["k"], g2["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o2, r2[0]) and torch.equal(l2, r2[1])
