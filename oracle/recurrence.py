"""The page's online-softmax recurrence and the partial-state merge, in float64.

TEST INFRASTRUCTURE ONLY (see oracle/attention.py): nothing on the product path
imports it. It exists so that the tests can check, on tiny inputs, the claim that
processing keys block by block reaches the same result as the full softmax, and so
that the merge of partial states used by a split over keys has a plain statement.

Source: page "编译器与内核" (Compilers and kernels), section
"FlashAttention 围绕 IO 改写算法", the recurrence display and the symbol list under it.
For one query row i, start from m_0 = -inf, l_0 = 0, o_0 = 0 in R^{d_v}; for each
key block B_t:
    b_t = max_{j in B_t} S_ij,     m_t = max(m_{t-1}, b_t),
    alpha_t = exp(m_{t-1} - m_t),
    l_t = alpha_t l_{t-1} + sum_{j in B_t} exp(S_ij - m_t),
    o_t = alpha_t o_{t-1} + sum_{j in B_t} exp(S_ij - m_t) v_j,
and after T blocks O_i = o_T / l_T. The page lets B_1..B_T partition the allowed
keys; a tiled kernel also meets blocks whose keys are all forbidden. Reading taken
here: such a block (and any block met while no allowed key has been seen, so that
m_t = -inf) leaves the state unchanged (alpha = 1, nothing added), which is the
value the recurrence has when the forbidden keys are simply left out of the
partition.

The merge of two partial states over disjoint key sets A and B follows from the same
recurrence (processing the keys of B after those of A, in one block):
    m = max(m_A, m_B), l = e^{m_A-m} l_A + e^{m_B-m} l_B, o = e^{m_A-m} o_A + e^{m_B-m} o_B.
The page "AI 编译器开发工程师…" (section on the reduction-vs-parallelism conflict in
softmax) describes splitting the reduction into segments whose partial results are
merged afterwards; its merge formula did not survive extraction, so the merge here is
derived from the recurrence above and pinned by the tests against the full softmax.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["State", "online_softmax_row", "merge_states", "finish"]


class State:
    """Running statistics of one query row: max m, normaliser l, numerator o."""

    __slots__ = ("m", "l", "o")

    def __init__(self, dv: int):
        self.m = -math.inf
        self.l = 0.0
        self.o = np.zeros(dv, dtype=np.float64)


def _step(state: State, s_blk: np.ndarray, v_blk: np.ndarray) -> None:
    """One block of the recurrence, in the page's order."""
    b_t = float(s_blk.max()) if s_blk.size else -math.inf
    m_t = max(state.m, b_t)
    if m_t == -math.inf:
        # no allowed key seen so far: alpha_t = 1 and the block adds nothing
        return
    alpha_t = math.exp(state.m - m_t)  # exp(-inf) = 0 on the first allowed block
    w = np.exp(s_blk - m_t)            # exp(S_ij - m_t), forbidden keys give 0
    state.l = alpha_t * state.l + float(w.sum())
    state.o = alpha_t * state.o + w @ v_blk
    state.m = m_t


def online_softmax_row(s_row, v, blocks) -> State:
    """Run the recurrence over `blocks` (a list of key-index arrays) for one row.

    s_row: [N] scores S_i. (already scaled and biased, -inf for forbidden keys);
    v: [N, dv]. Returns the final State (m_T, l_T, o_T).
    """
    s_row = np.asarray(s_row, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    st = State(v.shape[1])
    for blk in blocks:
        blk = np.asarray(blk, dtype=np.int64)
        _step(st, s_row[blk], v[blk])
    return st


def merge_states(a: State, b: State) -> State:
    """Merge the states of two disjoint key sets (see module docstring)."""
    out = State(a.o.shape[0])
    m = max(a.m, b.m)
    if m == -math.inf:
        return out
    ea = math.exp(a.m - m)
    eb = math.exp(b.m - m)
    out.m = m
    out.l = ea * a.l + eb * b.l
    out.o = ea * a.o + eb * b.o
    return out


def finish(st: State):
    """O_i = o_T / l_T and lse_i = m_T + ln l_T; (0, -inf) when no key was allowed."""
    if st.m == -math.inf:
        return np.zeros_like(st.o), -math.inf
    return st.o / st.l, st.m + math.log(st.l)
