"""GPU parity of the gradients over seeded random problem shapes: bf16 and fp16, the
matrix-core widths d, dv in {64, 128}, sequence length, causal mask, additive bias with a
sparse -inf mask, batch and head counts and both storage layouts, through the C ABI
against the fp64 gradient oracle on the same seeded inputs (the forward runs first, as a
training step would). The shapes are drawn once from a fixed seed.
"""

import numpy as np
import pytest

from exact_attention_35_amd import capi, workloads
from oracle import sdpa_backward_reference
from parity_util import check_grad

pytestmark = pytest.mark.gpu


def _cases(n=16, seed=35456):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "bf16" if rng.random() < 0.7 else "f16"
        d, dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
        N = int(rng.integers(1, 450))
        causal, bias = bool(rng.random() < 0.5), bool(rng.random() < 0.4)
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        layout = "bnhd" if rng.random() < 0.3 else "bhnd"
        out.append((i, dtype, d, dv, N, causal, bias, B, H, layout))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[f"r{c[0]}-{c[1]}-d{c[2]}-{c[3]}-n{c[4]}" for c in CASES])
def test_random_shape_gradients(gpu_device, case):
    import torch

    i, dtype, d, dv, N, causal, bias, B, H, layout = case
    w = workloads.workload(3).resized(B=B, H=H, N=N, d=d, dv=dv, causal=causal, bias=bias,
                                      mask_p=0.1 if bias else 0.0, dtype=dtype, layout=layout, seed=37000 + i)
    print(f"\n[random bwd] {case}", flush=True)
    inp = workloads.make_inputs(w, device="cpu")
    inp["do"] = workloads.make_grad_out(w, device="cpu")
    g = {}
    for n, t in inp.items():
        if t is None:
            g[n] = None
        elif layout == "bnhd" and n in ("q", "k", "v", "do"):
            g[n] = t.permute(0, 2, 1, 3).contiguous().to(gpu_device).permute(0, 2, 1, 3)  # [B, N, H, *] storage
        else:
            g[n] = t.to(gpu_device)
    out, lse = capi.fa_fwd(g["q"], g["k"], g["v"], bias=g["bias"], causal=causal)
    dq, dk, dv_ = capi.fa_bwd(g["q"], g["k"], g["v"], out, lse, g["do"], bias=g["bias"], causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv, (sq, sk, sv) = sdpa_backward_reference(inp["q"], inp["k"], inp["v"], inp["do"], inp["bias"],
                                                       causal, with_scales=True)
    check_grad(dq, rq, sq, f"dQ {case}", dtype=dtype)
    check_grad(dk, rk, sk, f"dK {case}", dtype=dtype)
    check_grad(dv_, rv, sv, f"dV {case}", dtype=dtype)
