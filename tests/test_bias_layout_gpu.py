"""GPU parity of the matrix-core forward with a bias whose rows are 16-byte aligned
(each lane loads its bias as 16-byte vectors) against the same logical bias in a layout
whose rows are not (element loads): the two must agree bitwise, and both match the fp64
oracle. Shapes reach ragged key and query tiles, causal masks, split plans (ranges that
start on odd tiles), broadcast, padded and rectangular bias, both 16-bit types, and
three of the width pairs.
"""

import numpy as np
import pytest
import torch

from exact_attention_35_amd import capi
from oracle import sdpa_reference
from parity_util import check_lse, check_out

pytestmark = pytest.mark.gpu


def _bias(shape, causal_off, gen):
    """fp32 N(0,1) bias with 10% of its entries -inf; key i + causal_off of row i kept."""
    bias = torch.randn(shape, generator=gen)
    bias[torch.rand(shape, generator=gen) < 0.1] = float("-inf")
    nq, nk = shape[-2], shape[-1]
    rows = torch.arange(nq)
    keep = (rows + causal_off).clamp(0, nk - 1)
    bias[..., rows, keep] = torch.randn(shape[:-2] + (nq,), generator=gen)
    return bias


def _padded(bias, pad, dev):
    """`bias` on the device in a buffer whose rows are nk + pad floats apart."""
    nk = bias.shape[-1]
    buf = torch.zeros(bias.shape[:-1] + (nk + pad,), dtype=torch.float32, device=dev)
    buf[..., :nk] = bias.to(dev)
    return buf[..., :nk]


CASES = [  # (d, dv, B, H, N_q, N_k, causal, bias shape ("bh", "1h", "11"), dtype)
    (64, 128, 1, 2, 1000, 1000, False, "1h", "bf16"),   # split plan, ragged tiles
    (64, 64, 2, 3, 512, 512, True, "11", "bf16"),       # broadcast bias, causal
    (64, 128, 1, 1, 2048, 2048, True, "11", "f16"),     # split plan, causal diagonal tiles
    (128, 64, 1, 4, 768, 768, False, "bh", "bf16"),     # the d = 128, dv = 64 variant
    (64, 128, 4, 32, 512, 512, False, "1h", "bf16"),    # no split: whole query tiles
    (64, 128, 1, 2, 300, 1200, True, "1h", "bf16"),     # rectangular, causal offset
    (64, 64, 1, 1, 100, 200, False, "11", "f16"),       # one partial query tile, 4 key tiles
]


@pytest.mark.parametrize("case", CASES, ids=[f"d{c[0]}-dv{c[1]}-b{c[2]}h{c[3]}-{c[4]}x{c[5]}-c{int(c[6])}-{c[7]}-{c[8]}"
                                             for c in CASES])
def test_aligned_and_unaligned_bias_rows_agree_and_match_oracle(gpu_device, case):
    d, dv, B, H, nq, nk, causal, bshape, dtype = case
    gen = torch.Generator().manual_seed(35100 + nq + 7 * nk + d + H)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    q = torch.randn(B, H, nq, d, generator=gen).to(tdt)
    k = torch.randn(B, H, nk, d, generator=gen).to(tdt)
    v = torch.randn(B, H, nk, dv, generator=gen).to(tdt)
    lead = {"bh": (B, H), "1h": (1, H), "11": (1, 1)}[bshape]
    bias = _bias(lead + (nq, nk), (nk - nq) if causal else 0, gen)
    dev = gpu_device
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    fwd = capi.fa_fwd if nq == nk else capi.fa_fwd_qk
    # rows nk + 4 floats apart: 16-byte aligned (vector loads); nk + 1 apart: not (element loads)
    staged, regs = _padded(bias, 4, dev), _padded(bias, 1, dev)
    assert staged.stride(2) % 4 == 0 and regs.stride(2) % 4 != 0
    o_s, l_s = fwd(qd, kd, vd, bias=staged, causal=causal)
    o_r, l_r = fwd(qd, kd, vd, bias=regs, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_r) and torch.equal(l_s, l_r), "vector and element bias loads differ"
    o_ref, l_ref, sc = sdpa_reference(q, k, v, bias, causal, with_scale=True)
    key = "bf16" if dtype == "bf16" else "f16_mfma"
    check_out(o_s, o_ref, key, str(case), scale=sc)
    check_lse(l_s, l_ref, str(case))
