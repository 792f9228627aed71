"""FLOP and byte accounting for the attention forward, and the roofline bound.

Host-side bookkeeping for the benchmark; no kernel arithmetic lives here.

Roofline, as stated on the page "编译器与内核" (Compilers and kernels), section
"屋顶线是上界，不是秒表": for a kernel with F floating-point operations and Q bytes
crossing the measured memory boundary, I = F/Q, the attainable throughput is
min(P_max, B_max * I), the time is at least max(F/P_max, Q/B_max), and the ridge is
P_max / B_max.

Traffic accounting for one head follows the page "AI Infra 第5章图解: 算子与运行时",
section "FlashAttention: Softmax 也能逐块算": the required traffic is reading Q, K, V
and writing O; a version that materialises the scores S and probabilities P in fp32
writes and reads each of them once more.
"""

from __future__ import annotations

__all__ = [
    "MI355X_PEAK_BF16_FLOPS", "MI355X_PEAK_F32_FLOPS", "MI355X_HBM_BYTES_PER_S",
    "allowed_pairs", "alg_flops", "alg_flops_bwd", "min_bytes", "min_bytes_bwd", "materialised_sp_bytes",
    "intensity", "roofline_bound", "ridge",
]

# MI355X published figures (vendor specification; the pages print none for AMD).
MI355X_PEAK_BF16_FLOPS = 2.5e15      # dense bf16 MFMA
MI355X_PEAK_F32_FLOPS = 157.3e12     # fp32 matrix / vector
MI355X_HBM_BYTES_PER_S = 8.0e12      # HBM3E


def allowed_pairs(N: int, causal: bool, Nq: int = None) -> int:
    """Query/key pairs per head that the mask allows (no bias mask counted). With Nq
    query rows against N keys, the causal mask lets row i see keys j <= i + N - Nq."""
    if Nq is None or Nq == N:
        return N * (N + 1) // 2 if causal else N * N
    if not causal:
        return Nq * N
    off = N - Nq
    # row i sees min(N, max(0, i + off + 1)) keys
    lo = max(0, -off)                 # first row that sees a key
    hi = min(Nq, N - off)             # rows below hi see fewer than N keys
    partial = sum(range(lo + off + 1, hi + off + 1)) if hi > lo else 0
    return partial + max(0, Nq - max(hi, lo)) * N


def alg_flops(B, H, N, d, dv, causal, pairs=None, Nq=None) -> int:
    """Algorithmic FLOPs: 2*d per pair for QK^T plus 2*dv per pair for PV.

    Softmax arithmetic is not counted. `pairs` overrides the per-head count (e.g. the
    allowed pairs of a sparse bias mask); Nq: query rows when they differ from N.
    """
    p = allowed_pairs(N, causal, Nq) if pairs is None else pairs
    return 2 * (d + dv) * p * B * H


def alg_flops_bwd(B, H, N, d, dv, causal, pairs=None) -> int:
    """Algorithmic FLOPs of the gradients: the five products per allowed pair,
    S = Q K^T (2d), dP = dO V^T (2dv), dV += P^T dO (2dv), dQ += dS K (2d) and
    dK += dS^T Q (2d), i.e. 2*(3d + 2dv); recomputing S and dP a second time (as a
    split into dK/dV and dQ passes does) is not counted."""
    p = allowed_pairs(N, causal) if pairs is None else pairs
    return 2 * (3 * d + 2 * dv) * p * B * H


def min_bytes_bwd(B, H, N, d, dv, elem_bytes, bias_bytes=0) -> int:
    """Minimum HBM bytes of the gradients: Q, K, V, O, dO and lse read once, dQ, dK,
    dV written once, and an optional bias read once."""
    return B * H * N * ((2 * d + 3 * dv) * elem_bytes + 4 + (2 * d + dv) * elem_bytes) + bias_bytes


def min_bytes(B, H, N, d, dv, elem_bytes, bias_bytes=0, lse_bytes=4, Nq=None) -> int:
    """Minimum HBM bytes: Q, K, V read once, O written once, lse written once,
    and an optional bias read once (`bias_bytes` is its total size). Nq: query rows
    (Q, O, lse) when they differ from the N keys (K, V)."""
    nq = N if Nq is None else Nq
    qkv = B * H * (nq * d + N * (d + dv)) * elem_bytes
    o = B * H * nq * dv * elem_bytes
    return qkv + o + B * H * nq * lse_bytes + bias_bytes


def materialised_sp_bytes(B, H, N, sp_elem_bytes=4) -> int:
    """Extra traffic of a version that writes S and P to memory and reads each back
    once: 2 matrices x (1 write + 1 read) x N*N elements per head."""
    return 2 * 2 * N * N * sp_elem_bytes * B * H


def intensity(flops, nbytes) -> float:
    return flops / nbytes


def ridge(p_max, b_max) -> float:
    return p_max / b_max


def roofline_bound(flops, nbytes, p_max, b_max):
    """(attainable FLOP/s, lower bound on time in s, which ceiling binds)."""
    i = flops / nbytes
    attain = min(p_max, b_max * i)
    t = max(flops / p_max, nbytes / b_max)
    return attain, t, ("compute" if p_max <= b_max * i else "memory")
