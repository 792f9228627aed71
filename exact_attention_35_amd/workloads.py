"""Seeded synthetic workloads for the attention forward and its gradients.

This module only draws inputs: it holds no part of the attention arithmetic, so the
tests can hand the very same tensors to the HIP path and to the CPU oracle.

Recipe (the same for every workload):
  * generator: numpy ``default_rng(seed)`` (PCG64);
  * draw order: Q, K, V, then bias values, then the mask's uniform draws;
  * each tensor is drawn as float32 standard normals in its *storage* layout and
    multiplied by its sigma; bf16 workloads round to bfloat16 (round to nearest
    even, via torch) — the oracle receives the rounded values;
  * the sparse mask sets a bias entry to -inf with probability `mask_p`,
    independently per (h, i, j) with i != j; diagonal entries keep their value, so
    every query row keeps at least one allowed key;
  * the upstream gradient dO of the gradient workloads is drawn separately
    (seed + 500000), N(0, 1) in the same storage layout and dtype as V.

The five workloads are the single fp32 head (N=256, d=64), the single bf16 causal head
of length 8192 and width 128 that the traffic accounting on the page
"AI Infra 第5章图解: 算子与运行时" (section "FlashAttention: Softmax 也能逐块算")
uses, a batched multi-head causal case in [B, N, H, d] storage, an additive fp32 bias
with a 10% sparse mask and d != dv, and a long causal sequence with peaked scores; and
one decoding step (a single query row per head against 8192 cached keys).
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_grad_out", "workload"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dv: int
    dtype: str            # "f32", "bf16" or "f16": dtype of Q, K, V and O
    layout: str           # "bhnd" (contiguous [B,H,N,*]) or "bnhd" ([B,N,H,*] storage)
    causal: bool
    bias: bool            # fp32 additive bias of shape [1, H, N, N] (broadcast over B)
    q_sigma: float = 1.0
    k_sigma: float = 1.0
    v_sigma: float = 1.0
    mask_p: float = 0.0   # probability that an off-diagonal bias entry is -inf
    seed: int = 0
    Nq: int = 0           # query rows when they differ from the N keys (0: N_q = N)

    @property
    def n_q(self) -> int:
        return self.Nq if self.Nq else self.N

    def resized(self, **kw) -> "Workload":
        """Same distribution and structure at other sizes (for CPU-sized parity cases)."""
        return replace(self, **kw)


WORKLOADS = {
    "fp32_single_head_n256_d64": Workload(
        "fp32_single_head_n256_d64", B=1, H=1, N=256, d=64, dv=64, dtype="f32",
        layout="bhnd", causal=False, bias=False, seed=35001),
    "bf16_causal_single_head_n8192_d128": Workload(
        "bf16_causal_single_head_n8192_d128", B=1, H=1, N=8192, d=128, dv=128,
        dtype="bf16", layout="bhnd", causal=True, bias=False, seed=35002),
    "bf16_causal_b4_h32_n4096_d128_bnhd": Workload(
        "bf16_causal_b4_h32_n4096_d128_bnhd", B=4, H=32, N=4096, d=128, dv=128,
        dtype="bf16", layout="bnhd", causal=True, bias=False, seed=35003),
    "bf16_bias_mask_b2_h16_n2048_d64_dv128": Workload(
        "bf16_bias_mask_b2_h16_n2048_d64_dv128", B=2, H=16, N=2048, d=64, dv=128,
        dtype="bf16", layout="bhnd", causal=False, bias=True, mask_p=0.1, seed=35004),
    "bf16_causal_long_h8_n32768_d128": Workload(
        "bf16_causal_long_h8_n32768_d128", B=1, H=8, N=32768, d=128, dv=128,
        dtype="bf16", layout="bhnd", causal=True, bias=False, q_sigma=2.0, k_sigma=2.0,
        seed=35005),
    # the tile-shape experiment of the general kernel (fp32, no mask: every query tile
    # streams every key and value once)
    "fp32_tile_sweep_h8_n4096_d64": Workload(
        "fp32_tile_sweep_h8_n4096_d64", B=1, H=8, N=4096, d=64, dv=64, dtype="f32",
        layout="bhnd", causal=False, bias=False, seed=35007),
    # one decoding step against a key/value cache: one query row per (b, h)
    "bf16_decode_b8_h32_nk8192_d128": Workload(
        "bf16_decode_b8_h32_nk8192_d128", B=8, H=32, N=8192, d=128, dv=128, dtype="bf16",
        layout="bhnd", causal=True, bias=False, seed=35006, Nq=1),
}

# The order the workloads are listed in (small fp32 case first, headline case second).
WORKLOAD_ORDER = list(WORKLOADS)

# The traffic sweep: causal bf16 heads of d = dv = 128 at a fixed B*H*N = 32768 rows, from
# 16 heads of 2048 to one head of 32768, with the headline's distribution (N(0, 1)). The
# pages' IO analysis of the blockwise method puts its K/V traffic at Theta(N^2 d^2 / M);
# at fixed B*H*N the quadratic term grows with N while the minimum bytes stay fixed.
for _h, _n in ((16, 2048), (8, 4096), (4, 8192), (2, 16384), (1, 32768)):
    _name = f"bf16_causal_sweep_h{_h}_n{_n}_d128"
    WORKLOADS[_name] = Workload(_name, B=1, H=_h, N=_n, d=128, dv=128, dtype="bf16", layout="bhnd",
                                causal=True, bias=False, seed=36000 + _n)
del _h, _n, _name


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[WORKLOAD_ORDER[name_or_index]]
    return WORKLOADS[name_or_index]


def _draw(rng, shape, sigma):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def make_inputs(w: Workload, device="cpu"):
    """Draw one workload's inputs. Returns a dict of torch tensors.

    q: logical [B, H, N_q, d]; k: logical [B, H, N, d]; v: logical [B, H, N, dv] — views
    whose storage follows `w.layout` ([B,N,H,*] storage gives non-contiguous [B,H,N,*]
    views). bias: None or fp32 [1, H, N_q, N] (broadcast over B, i.e. batch stride 0).
    """
    import torch

    rng = np.random.default_rng(w.seed)
    if w.layout == "bhnd":
        shp = lambda n, dd: (w.B, w.H, n, dd)         # noqa: E731
        to_logical = lambda t: t                      # noqa: E731
    elif w.layout == "bnhd":
        shp = lambda n, dd: (w.B, n, w.H, dd)         # noqa: E731
        to_logical = lambda t: t.permute(0, 2, 1, 3)  # noqa: E731
    else:
        raise ValueError(w.layout)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
    out = {}
    for name, n, dd, sig in (("q", w.n_q, w.d, w.q_sigma), ("k", w.N, w.d, w.k_sigma),
                             ("v", w.N, w.dv, w.v_sigma)):
        t = torch.from_numpy(_draw(rng, shp(n, dd), sig)).to(tdt)
        out[name] = to_logical(t.to(device))
    out["bias"] = None
    if w.bias:
        vals = _draw(rng, (1, w.H, w.n_q, w.N), 1.0)
        if w.mask_p > 0:
            u = rng.random(size=(1, w.H, w.n_q, w.N), dtype=np.float32)
            kill = u < np.float32(w.mask_p)
            idx = np.arange(min(w.n_q, w.N))
            kill[:, :, idx, idx] = False
            vals[kill] = -np.inf
        out["bias"] = torch.from_numpy(vals).to(device)
    return out


def make_grad_out(w: Workload, device="cpu"):
    """dO for the gradient workloads: logical [B, H, N, dv], same layout and dtype as V."""
    import torch

    rng = np.random.default_rng(w.seed + 500000)
    shape = (w.B, w.H, w.N, w.dv) if w.layout == "bhnd" else (w.B, w.N, w.H, w.dv)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
    t = torch.from_numpy(_draw(rng, shape, 1.0)).to(tdt).to(device)
    return t if w.layout == "bhnd" else t.permute(0, 2, 1, 3)
