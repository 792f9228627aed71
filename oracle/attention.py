"""Plain fp64 CPU oracle for the exact scaled-dot-product attention forward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
module; only the tests, the smoke check and the CPU-baseline leg of the benchmark do.
It shares no code, constants or helpers with the HIP library.

What it computes is the definition stated on the page "编译器与内核" (Compilers and
kernels), section "FlashAttention 围绕 IO 改写算法", first display equation and the
symbol list under it:

    S = Q K^T / sqrt(d) + C,   m_i = max_j S_ij,   l_i = sum_j exp(S_ij - m_i),
    P_ij = exp(S_ij - m_i) / l_i,   O = P V,

with Q, K in R^{N x d}, V in R^{N x d_v}, C in (R u {-inf})^{N x N} an additive bias
or mask where -inf forbids a key, and every query row having at least one allowed key.
The same page states that the tiled method computes the same mathematical function
(not the same bits), so the oracle is the definition itself: it materialises S and P
in float64 and never tiles keys.

Readings taken where the page is silent (each is listed in the design notes):
  * log-sum-exp: lse_i = m_i + ln(l_i) = ln sum_j exp(S_ij), natural log, over the
    scaled and biased scores;
  * d (the Q/K width) sets the scale even when d != d_v;
  * C is added after scaling and is not itself scaled;
  * causal means C_ij = -inf for j > i + (N_k - N_q): with N_q = N_k = N the square
    mask above the diagonal; with N_q query rows against N_k keys the rows are aligned
    to the end of the key sequence (query i is position N_k - N_q + i, so one query
    row against a long key sequence sees every key); a bias and the causal mask add;
  * a bias tensor may broadcast over batch (stride 0) or over heads;
  * a row with no allowed key violates the page's precondition; by default the oracle
    raises, and with ``allow_empty_rows=True`` it returns the convention O = 0,
    lse = -inf for that row (this convention is not fixed by the page: parity
    unpinned for that row).

Inputs are taken exactly as the GPU saw them (bf16 or fp32 values) and upcast to
float64; upcasting bf16 or fp32 to float64 is exact.

With ``with_scale=True`` the oracle also returns, per output element, the scale of the
rounding errors a 16-bit kernel makes, S_ik = sqrt(sum_j P_ij^2 v_jk^2) (the terms that
rounding the probabilities to 16 bits before P V multiplies), which sizes the 16-bit
parity bar. It is pinned in tests/test_oracle_error_scales.py against an emulation of
16-bit rounding, closed forms and planted kernel bugs.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["sdpa_reference", "sdpa_reference_rows", "EmptyRowError"]


class EmptyRowError(ValueError):
    """A query row has no allowed key (the definition assumes at least one)."""


def _as_f64(x) -> np.ndarray:
    # torch tensors (any dtype, incl. bfloat16) and numpy arrays are both accepted;
    # a bf16 torch tensor is first widened to fp32 (exact), then to fp64 (exact).
    if hasattr(x, "detach"):
        t = x.detach().cpu()
        if str(t.dtype) in ("torch.bfloat16", "torch.float16"):
            t = t.float()
        x = t.numpy()
    return np.asarray(x, dtype=np.float64)


def _row_block(qbh, kbh, vbh, c_rows, rows, causal, scale, allow_empty_rows, with_scale=False):
    """Rows `rows` of one (batch, head): the definition, written out in float64.

    c_rows is None or the bias rows already selected ([len(rows), N_k]).
    with_scale: also return the rounding-error scale of O (see `_error_scale`).
    """
    n_q = qbh.shape[0]
    # S = Q K^T / sqrt(d) + C  (C = bias + causal mask)
    s = (qbh[rows] @ kbh.T) * scale
    if c_rows is not None:
        s = s + c_rows
    if causal:
        keys = np.arange(kbh.shape[0])[None, :]
        s = np.where(keys > rows[:, None] + (kbh.shape[0] - n_q), -np.inf, s)
    # m_i = max_j S_ij
    m = s.max(axis=1, initial=-np.inf)  # max over no key at all: -inf (an empty row)
    empty = ~np.isfinite(m) & (m < 0)
    if empty.any() and not allow_empty_rows:
        raise EmptyRowError(f"{int(empty.sum())} query row(s) have no allowed key")
    m_safe = np.where(empty, 0.0, m)
    # exp(S_ij - m_i), with exp(-inf) = 0
    e = np.exp(s - m_safe[:, None])
    # l_i = sum_j exp(S_ij - m_i)
    ell = e.sum(axis=1)
    ell_safe = np.where(empty, 1.0, ell)
    # P_ij = exp(S_ij - m_i) / l_i ;  O = P V
    p = e / ell_safe[:, None]
    o = p @ vbh
    lse = m_safe + np.log(ell_safe)
    o[empty] = 0.0
    lse[empty] = -np.inf
    if with_scale:
        return o, lse, _error_scale(p, vbh)
    return o, lse


def _error_scale(p, vbh):
    """Scale of the rounding errors of a 16-bit computation of O (tolerances only).

    Not part of the result. A method that rounds each probability to a 16-bit type
    before the products P V (relative error at most u per term, independent from term
    to term) moves O_ik by sum_j delta_ij P_ij v_jk, whose size is set by the
    root-sum-square of the terms it multiplies:
        scale_ik = sqrt(sum_j P_ij^2 v_jk^2).
    The same scale sizes the rounding of partial outputs over key ranges (each a convex
    combination of its range's v_j, weighted by its share of the probability mass).
    """
    return np.sqrt((p ** 2) @ (vbh ** 2))


def _bias_slice(bias, b, h):
    if bias is None:
        return None
    # bias broadcasts to [B, H, N_q, N_k]
    bb = bias.shape[0]
    bh = bias.shape[1]
    return bias[b if bb > 1 else 0, h if bh > 1 else 0]


def sdpa_reference(q, k, v, bias=None, causal=False, *, row_chunk=2048,
                   allow_empty_rows=False, with_scale=False):
    """Exact attention forward of every (batch, head) in float64.

    q: [B, H, N_q, d], k: [B, H, N_k, d], v: [B, H, N_k, dv] (logical layout; any real
    dtype, torch or numpy; N_q = N_k = N in the square case). bias: None or
    [Bb, Hb, N_q, N_k] with Bb in {1, B} and Hb in {1, H}; -inf entries forbid keys.
    causal: add -inf for keys j > i + (N_k - N_q).
    Returns (O [B, H, N_q, dv], lse [B, H, N_q]) as float64 numpy arrays, and with
    `with_scale` a third item: the rounding-error scale of O ([B, H, N_q, dv], see
    `_error_scale`), used only to size test tolerances.
    Query rows are processed in chunks of `row_chunk`; rows are independent in the
    definition, so chunking rows changes nothing.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    bias = None if bias is None else _as_f64(bias)
    B, H, N, d = q.shape
    nk = k.shape[2]
    dv = v.shape[-1]
    if k.shape != (B, H, nk, d) or v.shape != (B, H, nk, dv):
        raise ValueError("q, k, v shapes disagree")
    if bias is not None and (bias.ndim != 4 or bias.shape[2:] != (N, nk)
                             or bias.shape[0] not in (1, B) or bias.shape[1] not in (1, H)):
        raise ValueError("bias must broadcast to [B, H, N_q, N_k]")
    scale = 1.0 / math.sqrt(d)
    out = np.empty((B, H, N, dv), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    err = np.empty((B, H, N, dv), dtype=np.float64) if with_scale else None
    for b in range(B):
        for h in range(H):
            cbh = _bias_slice(bias, b, h)
            for r0 in range(0, N, row_chunk):
                rows = np.arange(r0, min(N, r0 + row_chunk))
                c_rows = None if cbh is None else cbh[rows]
                res = _row_block(q[b, h], k[b, h], v[b, h], c_rows, rows, causal,
                                 scale, allow_empty_rows, with_scale)
                out[b, h, rows] = res[0]
                lse[b, h, rows] = res[1]
                if with_scale:
                    err[b, h, rows] = res[2]
    if with_scale:
        return out, lse, err
    return out, lse


def sdpa_reference_rows(q, k, v, bias, causal, b, h, rows, *, allow_empty_rows=False,
                        with_scale=False):
    """The same definition for selected query rows of one (batch, head).

    Used at sizes where the full N_q x N_k problem is too large for the CPU: each
    sampled row is computed on its own, exactly as in `sdpa_reference`.
    q is [B, H, N_q, *], k and v are [B, H, N_k, *] (torch or numpy, any layout; only the needed slices are
    converted); bias as in `sdpa_reference`. Returns (O [len(rows), dv], lse [len(rows)]),
    and with `with_scale` the rounding-error scale of those rows of O.
    """
    rows = np.asarray(rows, dtype=np.int64)
    qbh = _as_f64(q[b, h])
    kbh = _as_f64(k[b, h])
    vbh = _as_f64(v[b, h])
    d = qbh.shape[-1]
    c_rows = None
    if bias is not None:
        bb = bias.shape[0]
        bh = bias.shape[1]
        sl = bias[b if bb > 1 else 0, h if bh > 1 else 0]
        c_rows = _as_f64(sl[rows.tolist()])
    return _row_block(qbh, kbh, vbh, c_rows, rows, causal, 1.0 / math.sqrt(d),
                      allow_empty_rows, with_scale)
