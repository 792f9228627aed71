"""GPU parity of the general path (fp32, widths other than 64 and 128, and layouts the
matrix-core kernel does not take: bases or row strides not 16-byte aligned) and of the
fp16 matrix-core kernel, through the C ABI against the fp64 oracle on the same seeded
inputs."""

import numpy as np
import pytest

from exact_attention_35_amd import capi, workloads
from oracle import sdpa_reference
from parity_util import check_lse, check_out

pytestmark = pytest.mark.gpu


def _run(w, dev, place=None, rect=False):
    import torch

    inp = workloads.make_inputs(w, device="cpu")
    g = {n: (None if t is None else t.to(dev)) for n, t in inp.items()}
    if place:
        g.update({n: place(g[n]) for n in ("q", "k", "v")})
    fwd = capi.fa_fwd_qk if rect else capi.fa_fwd
    out, lse = fwd(g["q"], g["k"], g["v"], bias=g["bias"], causal=w.causal)
    torch.cuda.synchronize()
    o_ref, l_ref, sc = sdpa_reference(inp["q"], inp["k"], inp["v"], inp["bias"], w.causal, with_scale=True)
    _run.scale = sc  # the oracle's rounding-error scale of the last case (16-bit bars)
    return out, lse, o_ref, l_ref


CASES = [  # (dtype, d, dv, N, causal, bias)
    ("bf16", 96, 96, 300, True, False),
    ("bf16", 40, 72, 150, False, True),
    ("bf16", 256, 256, 130, True, False),
    ("bf16", 128, 128, 700, False, True),    # bias at d = dv = 128: the most registers in use
    ("bf16", 128, 128, 650, True, True),     # the same, causal, on a split plan
    ("f32", 1, 256, 64, True, False),
    ("f32", 256, 24, 100, False, True),
    ("f16", 17, 33, 97, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-d{c[1]}-dv{c[2]}-n{c[3]}" for c in CASES])
def test_other_dtypes_and_widths(gpu_device, case):
    dt, d, dv, N, causal, bias = case
    w = workloads.workload(3).resized(B=1, H=2, N=N, d=d, dv=dv, causal=causal, bias=bias, dtype=dt,
                                      mask_p=0.1 if bias else 0.0, seed=8000 + d + dv + N)
    print(f"\n[general] {case}", flush=True)
    out, lse, o_ref, l_ref = _run(w, gpu_device)
    check_out(out, o_ref, dt, str(case), scale=_run.scale)
    check_lse(lse, l_ref, str(case))


def _misaligned(t):
    # the same values in storage that starts one element past a 16-byte boundary
    import torch

    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    return v


def _padded_rows(t):
    # rows of d + 4 elements (not a multiple of 16 bytes for bf16 at d = 64)
    import torch

    B, H, N, d = t.shape
    buf = torch.zeros(B, H, N, d + 4, dtype=t.dtype, device=t.device)
    buf[..., :d] = t
    return buf[..., :d]


@pytest.mark.parametrize("place", [_misaligned, _padded_rows], ids=["base+2B", "rows+8B"])
def test_layouts_outside_the_matrix_core_kernel(gpu_device, place):
    w = workloads.workload(1).resized(H=2, N=500, d=64, dv=64)
    out, lse, o_ref, l_ref = _run(w, gpu_device, place=place)
    check_out(out, o_ref, "bf16", place.__name__, scale=_run.scale)
    check_lse(lse, l_ref, place.__name__)


def test_fp16_rectangular_decode(gpu_device):
    # d = dv = 128, aligned: the matrix-core kernel with fp16 operands
    w = workloads.workload(1).resized(H=3, N=500, Nq=3, dtype="f16")
    out, lse, o_ref, l_ref = _run(w, gpu_device, rect=True)
    check_out(out, o_ref, "f16_mfma", "decode fp16", scale=_run.scale)
    check_lse(lse, l_ref, "decode fp16")


F16_MFMA = [  # (d, dv, N, causal, bias, B, H): the matrix-core kernel with fp16 operands
    (128, 128, 1000, True, False, 1, 1),     # split plan, in-kernel merge
    (128, 128, 333, True, False, 1, 2),
    (64, 128, 555, False, True, 2, 3),       # bias with a sparse mask
    (128, 64, 777, True, False, 2, 4),
    (64, 64, 129, True, True, 1, 2),
    (128, 128, 700, False, True, 1, 2),      # bias at d = dv = 128: the most registers in use
    (128, 128, 650, True, True, 2, 1),       # the same with a causal mask and a split plan
]


@pytest.mark.parametrize("case", F16_MFMA, ids=[f"d{c[0]}-dv{c[1]}-n{c[2]}" for c in F16_MFMA])
def test_fp16_matrix_core_path(gpu_device, case):
    d, dv, N, causal, bias, B, H = case
    w = workloads.workload(3).resized(B=B, H=H, N=N, d=d, dv=dv, causal=causal, bias=bias, dtype="f16",
                                      mask_p=0.1 if bias else 0.0, seed=8500 + N)
    out, lse, o_ref, l_ref = _run(w, gpu_device)
    check_out(out, o_ref, "f16_mfma", str(case), scale=_run.scale)
    check_lse(lse, l_ref, str(case))


def test_fp16_constant_v_is_exact(gpu_device):
    # o/l of every split range is a convex combination of V rows: constant V comes back
    # exactly through the fp16 partials and the merge
    import torch

    w = workloads.workload(1).resized(N=1000, dtype="f16")
    inp = workloads.make_inputs(w)
    q, k = inp["q"].to(gpu_device), inp["k"].to(gpu_device)
    v = torch.full_like(q, 1.6875)
    out, _ = capi.fa_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert bool((out == 1.6875).all())


@pytest.mark.parametrize("tile", [1, 2, 3, 4])
def test_tile_shapes_of_the_experiment(gpu_device, tile, monkeypatch):
    # every (BM, BK) of the tile-shape experiment computes the same function
    w = workloads.workload(0).resized(H=2, N=300, causal=True)
    monkeypatch.setenv("FA_GENERIC_TILE", str(tile))
    out, lse, o_ref, l_ref = _run(w, gpu_device)
    check_out(out, o_ref, "f32", f"tile {tile}")
    check_lse(lse, l_ref, f"tile {tile}")
