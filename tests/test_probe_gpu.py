"""The measurement probes of include/fa_probe.h on the GPU: the streaming copy copies, the
matrix-core probe reports its FLOP count, the launch timer stamps each armed main-kernel
launch with an interval that lies inside the launch's own event bracket, without changing
what the launch computes, and the LDS and tile-body probes time every wave.
"""

import numpy as np
import pytest

from exact_attention_35_amd import capi, workloads

pytestmark = pytest.mark.gpu


def test_copy_probe_copies(gpu_device):
    import torch

    src = torch.arange(1 << 22, dtype=torch.float32, device=gpu_device)
    dst = torch.zeros_like(src)
    capi.fa_probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    odd = torch.arange(1000, dtype=torch.float32, device=gpu_device)   # a ragged tail: 4000 bytes
    dodd = torch.zeros_like(odd)
    capi.fa_probe_copy(odd, dodd)
    torch.cuda.synchronize()
    assert torch.equal(odd, dodd)


def test_mfma_probe_flops(gpu_device):
    import torch

    out = torch.full((8 * 256,), float("nan"), dtype=torch.float32, device=gpu_device)
    flops = capi.fa_probe_mfma(out, 8, 10)
    torch.cuda.synchronize()
    assert flops == 8 * 4 * 10 * 4 * 32768
    assert torch.isfinite(out).all()


def _fwd_setup(dev, name="bf16_causal_sweep_h8_n4096_d128"):
    import torch

    w = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(w, device="cpu")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    out = torch.empty(w.B, w.H, w.N, w.dv, dtype=q.dtype, device=dev)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev)
    return q, k, v, out, lse


def test_launch_timer_stamps_inside_event_bracket(gpu_device):
    import torch

    q, k, v, out, lse = _fwd_setup(gpu_device)
    stream = torch.cuda.current_stream(gpu_device)
    call = lambda: capi.fa_fwd(q, k, v, causal=True, out=out, lse=lse, stream=stream)
    call()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()

    n = 12
    brackets = []
    capi.fa_probe_timer_arm(n)
    for _ in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        brackets.append((e0, e1))
    stamps = np.array(capi.fa_probe_timer_read(n))
    torch.cuda.synchronize()
    outer = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in brackets])
    print(f"kernel stamps us: median {np.median(stamps):.2f}; event brackets us: median {np.median(outer):.2f}")
    assert stamps.shape == (n,) and (stamps > 0).all()
    # the kernel's own interval is a sub-interval of the bracket around its launch
    assert (stamps <= outer * 1.01 + 1.0).all(), (stamps, outer)
    # timing a launch does not change what it computes
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    # after a read the timer is disarmed: further launches take no events
    call()
    assert capi.fa_probe_timer_read(0) == []


def test_launch_timer_count_mismatch_is_an_error(gpu_device):
    import torch

    q, k, v, out, lse = _fwd_setup(gpu_device, "bf16_causal_sweep_h16_n2048_d128")
    capi.fa_probe_timer_arm(3)
    capi.fa_fwd(q, k, v, causal=True, out=out, lse=lse)
    capi.fa_fwd(q, k, v, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    with pytest.raises(capi.FaError):
        capi.fa_probe_timer_read(3)      # only two of the three armed launches happened
    assert len(capi.fa_probe_timer_read(2)) == 2


def test_issue_probe_times_every_working_wave(gpu_device):
    # one MFMA wave per SIMD: 64 workgroups of 4 waves, every wave times its loop; a
    # 32x32x16 MFMA holds the matrix core at least 32 shader cycles
    cyc, rt, waves = capi.fa_probe_issue(0, 2, 0, 64, 500)
    assert len(cyc) == 64 * 4 and all(r > 0 for r in rt)
    per_mfma = sum(cyc) / len(cyc) / (2 * 500)
    assert 30.0 <= per_mfma < 200.0, per_mfma
    # roles with idle halves: only the working waves report
    cyc, rt, waves = capi.fa_probe_issue(2, 0, 0, 64, 200)
    assert len(cyc) == 64 * 4 and all(w % 8 < 4 for w in waves)
    cyc, rt, waves = capi.fa_probe_issue(3, 0, 1, 64, 200)
    assert len(cyc) == 64 * 4 and all(w % 8 >= 4 for w in waves)
    cyc, rt, waves = capi.fa_probe_issue(1, 0, 0, 64, 200)
    assert len(cyc) == 64 * 8


def test_read_probe_reads_and_checks_its_sink(gpu_device):
    import torch

    cus = torch.cuda.get_device_properties(gpu_device).multi_processor_count
    src = torch.arange(1 << 22, dtype=torch.int32, device=gpu_device)   # 16 MiB, nonzero words
    sink = torch.full((16 * cus,), -1, dtype=torch.int32, device=gpu_device)
    capi.fa_probe_read(src, sink)
    torch.cuda.synchronize()
    grid = min((src.numel() // 4 + 255) // 256, 16 * cus)
    assert (sink[:grid] != -1).all()        # every workgroup wrote its word
    assert (sink[grid:] == -1).all()        # nothing past the grid
    with pytest.raises(capi.FaError):
        capi.fa_probe_read(src, sink[:1])   # a sink smaller than the grid is refused


def test_lds_probe_times_every_wave(gpu_device):
    import torch

    cus = torch.cuda.get_device_properties(gpu_device).multi_processor_count
    for mode in range(5):
        cyc, rt, ms = capi.fa_probe_lds(mode, 2 * cus, 50)
        assert len(cyc) == 2 * cus * 4 and all(c > 0 for c in cyc) and all(r > 0 for r in rt) and ms > 0
        # eight waves per CU move 8 * 50 * 8 * 64 * width bytes; no LDS serves 1 KiB per clock
        width = (16, 8, 8, 4, 16)[mode]
        rate = 8 * 50 * 8 * 64 * width / (sum(cyc) / len(cyc))
        assert 0 < rate < 1024, (mode, rate)


def test_tile_probe_times_every_wave(gpu_device):
    import torch

    cus = torch.cuda.get_device_properties(gpu_device).multi_processor_count
    src = torch.zeros(1 << 18, dtype=torch.uint8, device=gpu_device)
    for copies in (0, 1):
        cyc, rt, ms = capi.fa_probe_tile(copies, 117, 2 * cus, 20, src)
        assert len(cyc) == 2 * cus * 4 and all(r > 0 for r in rt)
        # a SIMD's two waves issue 64 MFMAs per tile pair, 32 cycles each at least: the
        # launch lasts at least that long at the waves' clock
        mhz = 100.0 * sum(cyc) / sum(rt)
        per_pair = ms * 1e3 * mhz / 20
        assert 2048 <= per_pair < 20000, (copies, per_pair)
    with pytest.raises(capi.FaError):
        capi.fa_probe_tile(1, 117, 1, 1, src[:1024])   # the copy source must hold 256 KiB
