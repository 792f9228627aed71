"""Plain fp64 CPU oracle for the gradients of the exact attention forward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
module; only the tests and the benchmark's CPU-baseline leg do. It shares no code,
constants or helpers with the HIP library.

The page "编译器与内核" (Compilers and kernels), section "FlashAttention 围绕 IO 改写算法",
notes that the backward pass can recompute the score and probability blocks instead of
keeping them; it does not print the gradient formulas. They follow from the forward
definition of the same section,

    S = Q K^T / sqrt(d) + C,   P = rowsoftmax(S),   O = P V,

by the chain rule, for an upstream gradient dO of O:

    dV = P^T dO                               (O is linear in V)
    dP = dO V^T                               (O is linear in P)
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)   (Jacobian of one softmax row)
    dQ = dS K / sqrt(d),   dK = dS^T Q / sqrt(d)

C (bias and mask) is a constant of the problem: no gradient is formed for it. Keys a
row may not use have P_ij = 0, so they receive nothing. The oracle forms P from the
definition (it does not reuse a saved log-sum-exp), materialises S, P, dP and dS in
float64 and never tiles keys. Rows are processed in chunks (their contributions to dK
and dV are summed chunk after chunk in float64); rows are independent in the
definition, so chunking only changes the fp64 rounding order of those sums.

Readings (each is listed in the design notes): the same ones as the forward oracle
(scale 1/sqrt(d) with d the Q/K width; C added after scaling; causal is top-left
aligned; bias and mask add; bias broadcasts over batch or heads). A row with no
allowed key has no gradient (dQ row = 0, and it adds nothing to dK, dV): a
convention, parity unpinned.

With ``with_scales=True`` the oracle also returns the rounding-error scales sq, sk, sv of
every gradient element (the root-sum-square of the terms that 16-bit roundings of P, dS
and O multiply, plus the shared error of D_i = dO_i . O_i), which size the gradient
parity bar; they are pinned in tests/test_oracle_error_scales.py against an emulation of
16-bit arithmetic and against planted slips in their formulas.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import EmptyRowError, _as_f64, _bias_slice

__all__ = ["sdpa_backward_reference", "sdpa_backward_reference_sampled"]


def _probabilities(qbh, kbh, c_rows, rows, causal, scale, allow_empty_rows):
    """P for rows `rows` of one (batch, head), from the forward definition."""
    s = (qbh[rows] @ kbh.T) * scale
    if c_rows is not None:
        s = s + c_rows
    if causal:
        keys = np.arange(kbh.shape[0])[None, :]
        s = np.where(keys > rows[:, None], -np.inf, s)
    m = s.max(axis=1, initial=-np.inf)  # max over no key at all: -inf (an empty row)
    empty = ~np.isfinite(m) & (m < 0)
    if empty.any() and not allow_empty_rows:
        raise EmptyRowError(f"{int(empty.sum())} query row(s) have no allowed key")
    e = np.exp(s - np.where(empty, 0.0, m)[:, None])
    ell = e.sum(axis=1)
    p = e / np.where(empty, 1.0, ell)[:, None]
    p[empty] = 0.0
    return p


def _row_block_grads(qbh, kbh, vbh, dobh, c_rows, rows, causal, scale, allow_empty_rows,
                     with_scales=False):
    """dQ rows and the rows' contributions to dK, dV (all keys) for one (b, h).

    with_scales: also the rows' contributions to the rounding-error scales (see
    `_error_scales`), returned as a fourth item (sq rows, sk2 part, sv2 part)."""
    p = _probabilities(qbh, kbh, c_rows, rows, causal, scale, allow_empty_rows)
    do = dobh[rows]
    dv_part = p.T @ do                                # dV = P^T dO
    dp = do @ vbh.T                                   # dP = dO V^T
    ds = p * (dp - (p * dp).sum(axis=1)[:, None])     # softmax Jacobian, row by row
    dq = (ds @ kbh) * scale                           # dQ = dS K / sqrt(d)
    dk_part = (ds.T @ qbh[rows]) * scale              # dK = dS^T Q / sqrt(d)
    if not with_scales:
        return dq, dk_part, dv_part
    return dq, dk_part, dv_part, _error_scales(p, ds, qbh[rows], kbh, vbh, do, scale)


# Rounding-error scales of a 16-bit gradient computation (tolerances only; not part of
# the result). A rounded operand adds to a sum an error proportional to its term;
# independent roundings add in quadrature, so each gradient element gets the
# root-sum-square of its terms, plus the term of D_i = dO_i . O_i, whose error (O is
# given in 16 bits) is proportional to A_i = sum_k |dO_ik O_ik| and is shared by every
# key of row i (so it enters dQ_i in full, and dK_j in quadrature over rows):
#     sv^2 = (P^2)^T (dO^2),
#     sk^2 = scale^2 (dS^2 + (P A)^2)^T (Q^2),
#     sq   = scale (sqrt((dS^2 + (u P A)^2) (K^2)) + A |P K|).
# In sq, the dS that a kernel rounds carries D's error (up to u A_i P_ij, u = 2^-8 the
# unit roundoff of bf16, the coarser 16-bit type), so its rounding scales with
# |dS| + u P A; that second-order term matters only where P K cancels.

def _d_error_scale(o, do):
    """A_i = sum_k |dO_ik O_ik|: the size of D_i's error per unit of relative error in O."""
    return (np.abs(do) * np.abs(o)).sum(axis=1)


def _dq_scale(p, ds, kbh, a, scale):
    """sq for rows with probabilities p and dS ds over all keys."""
    u = 2.0 ** -8
    return scale * (np.sqrt((ds ** 2 + (u * p * a[:, None]) ** 2) @ kbh ** 2) + a[:, None] * np.abs(p @ kbh))


def _dkdv_scales(p, ds, q_rows, a, do, scale):
    """The rows' contributions to sk^2 and sv^2 of the key columns that p and ds hold."""
    sk2 = scale ** 2 * ((ds ** 2 + (p * a[:, None]) ** 2).T @ q_rows ** 2)
    sv2 = (p ** 2).T @ do ** 2
    return sk2, sv2


def _error_scales(p, ds, q_rows, kbh, vbh, do, scale):
    """sq of the rows, and the rows' contributions to sk^2 and sv^2 (all keys)."""
    a = _d_error_scale(p @ vbh, do)
    return (_dq_scale(p, ds, kbh, a, scale),) + _dkdv_scales(p, ds, q_rows, a, do, scale)


def _check_shapes(q, k, v, dout, bias):
    B, H, N, d = q.shape
    dv = v.shape[-1]
    if k.shape != (B, H, N, d) or v.shape != (B, H, N, dv) or dout.shape != (B, H, N, dv):
        raise ValueError("q, k, v, dout shapes disagree")
    if bias is not None and (bias.ndim != 4 or bias.shape[2:] != (N, N)
                             or bias.shape[0] not in (1, B) or bias.shape[1] not in (1, H)):
        raise ValueError("bias must broadcast to [B, H, N, N]")
    return B, H, N, d, dv


def sdpa_backward_reference(q, k, v, dout, bias=None, causal=False, *, row_chunk=1024,
                            allow_empty_rows=False, with_scales=False):
    """dQ, dK, dV of every (batch, head) in float64.

    q: [B, H, N, d], k: [B, H, N, d], v and dout: [B, H, N, dv] (logical layout; any real
    dtype, torch or numpy). bias and causal as in `sdpa_reference`.
    Returns (dQ [B,H,N,d], dK [B,H,N,d], dV [B,H,N,dv]) as float64 numpy arrays, and with
    `with_scales` a fourth item: the rounding-error scales (sq, sk, sv) of the same
    shapes, used only to size test tolerances (see `_error_scales`).
    """
    q, k, v, dout = (_as_f64(x) for x in (q, k, v, dout))
    bias = None if bias is None else _as_f64(bias)
    B, H, N, d, dvw = _check_shapes(q, k, v, dout, bias)
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros((B, H, N, d))
    dk = np.zeros((B, H, N, d))
    dv = np.zeros((B, H, N, dvw))
    if with_scales:
        sq, sk2, sv2 = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    for b in range(B):
        for h in range(H):
            cbh = _bias_slice(bias, b, h)
            for r0 in range(0, N, row_chunk):
                rows = np.arange(r0, min(N, r0 + row_chunk))
                c_rows = None if cbh is None else cbh[rows]
                res = _row_block_grads(q[b, h], k[b, h], v[b, h], dout[b, h], c_rows,
                                       rows, causal, scale, allow_empty_rows, with_scales)
                dq[b, h, rows] = res[0]
                dk[b, h] += res[1]
                dv[b, h] += res[2]
                if with_scales:
                    sq[b, h, rows] = res[3][0]
                    sk2[b, h] += res[3][1]
                    sv2[b, h] += res[3][2]
    if with_scales:
        return dq, dk, dv, (sq, np.sqrt(sk2), np.sqrt(sv2))
    return dq, dk, dv


def sdpa_backward_reference_sampled(q, k, v, dout, bias, causal, b, h, rows, keys, *,
                                    row_chunk=1024, with_scales=False):
    """dQ at query rows `rows` and dK, dV at key rows `keys` of one (batch, head).

    For sizes where the full gradients are too large for the CPU: dQ of a row needs only
    that row; dK and dV of a key need every row's probability of it, so all rows are
    formed chunk by chunk (S and P of each row in full, for its normaliser, and O = P V
    for D_i = dO_i . O_i, which equals sum_k P_ik dP_ik) and dP, dS are formed only in
    the sampled key columns. Under the causal mask, rows i see keys j <= i only, so a
    chunk of rows needs no key past its last row, and rows before the first sampled key
    add nothing to it (their probabilities of it are 0). Same definition as
    `sdpa_backward_reference`.
    Returns (dQ [len(rows), d], dK [len(keys), d], dV [len(keys), dv]).
    """
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    qbh, kbh, vbh, dobh = (_as_f64(x[b, h]) for x in (q, k, v, dout))
    N, d = qbh.shape
    scale = 1.0 / math.sqrt(d)
    sl = None
    if bias is not None:
        sl = bias[b if bias.shape[0] > 1 else 0, h if bias.shape[1] > 1 else 0]
    c_of = (lambda r, nk: None) if sl is None else (lambda r, nk: _as_f64(sl[r.tolist()])[:, :nk])
    res = _row_block_grads(qbh, kbh, vbh, dobh, c_of(rows, N), rows, causal, scale, False, with_scales)
    dq = res[0]
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), vbh.shape[1]))
    sk2, sv2 = np.zeros_like(dk), np.zeros_like(dv)
    first = int(keys.min()) if len(keys) else N
    for r0 in range(0, N, row_chunk):
        rr = np.arange(r0, min(N, r0 + row_chunk))
        if causal and rr[-1] < first:
            continue
        nk = int(rr[-1]) + 1 if causal else N    # keys any of these rows may see
        sel = np.nonzero(keys < nk)[0]
        p = _probabilities(qbh, kbh[:nk], c_of(rr, nk), rr, causal, scale, False)
        o = p @ vbh[:nk]
        do = dobh[rr]
        dd = (do * o).sum(axis=1)                    # D_i = dO_i . O_i
        pk = p[:, keys[sel]]
        dpk = do @ vbh[keys[sel]].T                  # dP in the sampled columns
        dsk = pk * (dpk - dd[:, None])               # dS in the sampled columns
        dv[sel] += pk.T @ do
        dk[sel] += (dsk.T @ qbh[rr]) * scale
        if with_scales:
            k2, v2 = _dkdv_scales(pk, dsk, qbh[rr], _d_error_scale(o, do), do, scale)
            sk2[sel] += k2
            sv2[sel] += v2
    if with_scales:
        return dq, dk, dv, (res[3][0], np.sqrt(sk2), np.sqrt(sv2))
    return dq, dk, dv
