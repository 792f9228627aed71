"""GPU parity of the forward over seeded random problem shapes: element type, head widths
(on and off the matrix-core kernel), N_q and N_k (equal or not), causal mask, additive
bias with a sparse -inf mask, batch and head counts, and both storage layouts, each
through the C ABI against the fp64 oracle on the same seeded inputs. The shapes are
drawn once from a fixed seed, so the cases are the same on every run.
"""

import numpy as np
import pytest

from exact_attention_35_amd import capi, workloads
from oracle import sdpa_reference
from parity_util import check_lse, check_out

pytestmark = pytest.mark.gpu


def _cases(n=36, seed=35123):
    rng = np.random.default_rng(seed)
    widths = [16, 32, 48, 64, 80, 96, 128, 192, 256]
    out = []
    for i in range(n):
        dtype = ["bf16", "bf16", "f16", "f32"][rng.integers(4)]
        if rng.random() < 0.5:  # half the cases on the matrix-core widths
            d, dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
        else:
            d, dv = int(rng.choice(widths)), int(rng.choice(widths))
        nk = int(rng.integers(1, 521))
        nq = nk if rng.random() < 0.6 else int(rng.integers(1, 521))
        causal, bias = bool(rng.random() < 0.5), bool(rng.random() < 0.4)
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 5))
        layout = "bnhd" if rng.random() < 0.3 else "bhnd"
        out.append((i, dtype, d, dv, nq, nk, causal, bias, B, H, layout))
    return out


CASES = _cases()


def _path_dtype(dtype, d, dv):
    # the tolerance of the path the call takes: 16-bit inputs at d, dv in {64, 128} run on
    # the matrix cores (P rounded to 16 bits), everything else in fp32 arithmetic
    on_mfma = dtype in ("bf16", "f16") and d in (64, 128) and dv in (64, 128)
    if dtype == "f16":
        return "f16_mfma" if on_mfma else "f16"
    return dtype


@pytest.mark.parametrize("case", CASES, ids=[f"r{c[0]}-{c[1]}-d{c[2]}-{c[3]}-q{c[4]}-k{c[5]}" for c in CASES])
def test_random_shape(gpu_device, case):
    import torch

    i, dtype, d, dv, nq, nk, causal, bias, B, H, layout = case
    w = workloads.workload(3).resized(B=B, H=H, N=nk, Nq=nq, d=d, dv=dv, causal=causal, bias=bias,
                                      mask_p=0.1 if bias else 0.0, dtype=dtype, layout=layout, seed=36000 + i)
    print(f"\n[random] {case}", flush=True)
    inp = workloads.make_inputs(w, device="cpu")
    g = {}
    for n, t in inp.items():
        if t is None:
            g[n] = None
        elif layout == "bnhd" and n in ("q", "k", "v"):
            g[n] = t.permute(0, 2, 1, 3).contiguous().to(gpu_device).permute(0, 2, 1, 3)  # [B, N, H, *] storage
        else:
            g[n] = t.to(gpu_device)
    bias_t = None if g["bias"] is None else g["bias"].expand(B, H, nq, nk)
    out, lse = capi.fa_fwd_qk(g["q"], g["k"], g["v"], bias=bias_t, causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref, sc = sdpa_reference(inp["q"], inp["k"], inp["v"], inp["bias"], causal, allow_empty_rows=True,
                                      with_scale=True)
    check_out(out, o_ref, _path_dtype(dtype, d, dv), str(case), scale=sc)
    check_lse(lse, l_ref, str(case))
