"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

None of these tests retypes the oracle's formula: each compares it with a different
route to the same number — exact rational arithmetic, closed forms, a worked example
from the pages, scalar brute force without the max shift, the page's block recurrence,
or invariants that any correct implementation satisfies. Each is chosen so that a
plausible slip (dropped or wrong scale, sign, transposed operand, wrong mask
direction, wrong log base, V index mix-up) fails at least one of them.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (EmptyRowError, finish, merge_states, online_softmax_row,
                    sdpa_reference, sdpa_reference_rows)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _scores(q, k, bias, causal):
    """S for one (b, h) in fp64 (used only to feed the recurrence tests)."""
    d = q.shape[-1]
    s = q @ k.T / math.sqrt(d)
    if bias is not None:
        s = s + bias
    if causal:
        n = s.shape[0]
        s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
    return s


# ---------------------------------------------------------------------------
# 1. exact rational arithmetic (closed form with nonzero Q and a scale that matters)
# ---------------------------------------------------------------------------

def _rational_case(seed, n=5, d=4, dv=3, masked_frac=0.3, causal=False):
    """Q, K chosen so that S_ij = ln w_j exactly when the scale 1/sqrt(d) is applied.

    q_i = (sqrt(d), 0, ...), k_j = (ln w_j, 0, ...) gives q_i.k_j / sqrt(d) = ln w_j.
    A bias C_ij = ln c_ij (or -inf) multiplies the weights: weight_ij = w_j * c_ij.
    Then O_i = sum_j weight_ij v_j / sum_j weight_ij is an exact rational.
    """
    rng = _rng(seed)
    w = rng.integers(1, 10, size=n)
    c = rng.integers(1, 10, size=(n, n)).astype(object)
    kill = rng.random((n, n)) < masked_frac
    for i in range(n):
        kill[i, i] = False
    v = rng.integers(-9, 10, size=(n, dv))
    q = np.zeros((1, 1, n, d))
    q[0, 0, :, 0] = math.sqrt(d)
    k = np.zeros((1, 1, n, d))
    k[0, 0, :, 0] = np.log(w)
    bias = np.log(np.array(c, dtype=np.float64))
    bias[kill] = -np.inf
    exp_o = np.zeros((n, dv), dtype=object)
    exp_lse = np.zeros(n)
    for i in range(n):
        num = [Fraction(0)] * dv
        den = Fraction(0)
        for j in range(n):
            if kill[i, j] or (causal and j > i):
                continue
            wt = Fraction(int(w[j])) * Fraction(int(c[i, j]))
            den += wt
            for t in range(dv):
                num[t] += wt * int(v[j, t])
        for t in range(dv):
            exp_o[i, t] = num[t] / den
        exp_lse[i] = math.log(den)
    return (q, k, v.astype(np.float64)[None, None], bias[None, None], exp_o, exp_lse)


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("causal", [False, True])
def test_exact_rationals_with_scale_bias_and_mask(seed, causal):
    q, k, v, bias, exp_o, exp_lse = _rational_case(seed, causal=causal)
    o, lse = sdpa_reference(q, k, v, bias, causal)
    ref = np.array([[float(x) for x in row] for row in exp_o])
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], exp_lse, rtol=1e-14, atol=1e-14)


def test_exact_rationals_d_sets_scale_not_dv():
    # d = 16 (scale 1/4) and dv = 2: a scale taken from dv would give 1/sqrt(2)
    q, k, v, bias, exp_o, exp_lse = _rational_case(99, n=6, d=16, dv=2)
    o, lse = sdpa_reference(q, k, v, bias, False)
    ref = np.array([[float(x) for x in row] for row in exp_o])
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], exp_lse, rtol=1e-14)


# ---------------------------------------------------------------------------
# 2. scalar brute force on tiny random inputs (no max shift, exact summation)
# ---------------------------------------------------------------------------

def _brute(q, k, v, c, causal):
    """Pure-Python loops: weights exp(S_ij) with no max subtraction, fsum sums."""
    n, d = len(q), len(q[0])
    dv = len(v[0])
    o = [[0.0] * dv for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        wts = []
        for j in range(n):
            if causal and j > i:
                wts.append(0.0)
                continue
            cij = c[i][j] if c is not None else 0.0
            if cij == -math.inf:
                wts.append(0.0)
                continue
            s = math.fsum(q[i][t] * k[j][t] for t in range(d)) / math.sqrt(d) + cij
            wts.append(math.exp(s))
        tot = math.fsum(wts)
        for t in range(dv):
            o[i][t] = math.fsum(wts[j] * v[j][t] for j in range(n)) / tot
        lse[i] = math.log(tot)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("seed", range(20))
def test_brute_force_tiny(seed):
    rng = _rng(1000 + seed)
    n = int(rng.integers(1, 7))
    d = int(rng.integers(1, 6))
    dv = int(rng.integers(1, 6))
    causal = bool(seed % 2)
    use_bias = seed % 3 != 0
    q = rng.standard_normal((1, 1, n, d))
    k = rng.standard_normal((1, 1, n, d))
    v = rng.standard_normal((1, 1, n, dv))
    bias = None
    if use_bias:
        bias = rng.standard_normal((1, 1, n, n))
        kill = rng.random((n, n)) < 0.3
        kill[np.arange(n), np.arange(n)] = False
        bias[0, 0][kill] = -np.inf
    o, lse = sdpa_reference(q, k, v, bias, causal)
    bo, bl = _brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                    None if bias is None else bias[0, 0].tolist(), causal)
    np.testing.assert_allclose(o[0, 0], bo, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], bl, rtol=1e-13, atol=1e-13)


def test_all_row_valid_masks_4x4():
    """Every one of the 15**4 = 50625 masks of a 4x4 problem with >=1 allowed key
    per row, batched over B; rows are checked against scalar brute force."""
    rng = _rng(7)
    n, d, dv = 4, 3, 2
    q1 = rng.standard_normal((n, d))
    k1 = rng.standard_normal((n, d))
    v1 = rng.standard_normal((n, dv))
    subsets = [s for s in range(1, 16)]          # nonempty subsets of 4 keys, as bits
    masks = np.array(list(itertools.product(subsets, repeat=n)))   # [50625, 4]
    nb = masks.shape[0]
    bits = (masks[:, :, None] >> np.arange(n)[None, None, :]) & 1  # [nb, i, j]
    bias = np.where(bits == 1, 0.0, -np.inf)[:, None]             # [nb, 1, 4, 4]
    q = np.broadcast_to(q1, (nb, 1, n, d))
    k = np.broadcast_to(k1, (nb, 1, n, d))
    v = np.broadcast_to(v1, (nb, 1, n, dv))
    o, lse = sdpa_reference(q, k, v, bias, False)
    # brute force per (row, subset): 60 distinct row results
    table_o = {}
    table_l = {}
    for i in range(n):
        for s in subsets:
            c = [[-math.inf] * n for _ in range(n)]
            for j in range(n):
                if (s >> j) & 1:
                    c[i][j] = 0.0
            for r in range(n):
                if r != i:
                    c[r][r] = 0.0
            bo, bl = _brute(q1.tolist(), k1.tolist(), v1.tolist(), c, False)
            table_o[i, s] = bo[i]
            table_l[i, s] = bl[i]
    exp_o = np.stack([np.stack([table_o[i, masks[b, i]] for i in range(n)])
                      for b in range(nb)])
    exp_l = np.array([[table_l[i, masks[b, i]] for i in range(n)] for b in range(nb)])
    np.testing.assert_allclose(o[:, 0], exp_o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[:, 0], exp_l, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# 3. the page's block recurrence reaches the full softmax (tiny inputs)
# ---------------------------------------------------------------------------

def _partitions(n, rng, kinds):
    out = []
    idx = np.arange(n)
    for bs in range(1, n + 1):                         # every contiguous block size
        out.append([idx[i:i + bs] for i in range(0, n, bs)])
    for _ in range(kinds):                             # random partitions, any order
        perm = rng.permutation(n)
        cuts = np.sort(rng.choice(np.arange(1, n), size=rng.integers(0, n), replace=False))
        out.append(np.split(perm, cuts))
    return out


@pytest.mark.parametrize("seed", range(6))
def test_online_recurrence_equals_full_softmax(seed):
    rng = _rng(2000 + seed)
    n, d, dv = 9, 5, 3
    q = rng.standard_normal((n, d)) * 2.0
    k = rng.standard_normal((n, d)) * 2.0
    v = rng.standard_normal((n, dv))
    bias = rng.standard_normal((n, n))
    # kill the first 4 keys for rows 5..8 so contiguous blocks can be fully masked
    bias[5:, :4] = -np.inf
    causal = bool(seed % 2)
    o, lse = sdpa_reference(q[None, None], k[None, None], v[None, None],
                            bias[None, None], causal)
    s = _scores(q, k, bias, causal)
    for blocks in _partitions(n, rng, kinds=25):
        for i in range(n):
            oi, li = finish(online_softmax_row(s[i], v, blocks))
            np.testing.assert_allclose(oi, o[0, 0, i], rtol=1e-13, atol=1e-13)
            assert abs(li - lse[0, 0, i]) < 1e-13 * max(1.0, abs(li))


@pytest.mark.parametrize("seed", range(4))
def test_merge_of_disjoint_states(seed):
    rng = _rng(3000 + seed)
    n, dv = 11, 4
    s = rng.standard_normal(n) * 3.0
    s[rng.random(n) < 0.3] = -np.inf
    s[0] = 0.5
    v = rng.standard_normal((n, dv))
    full_o, full_l = finish(online_softmax_row(s, v, [np.arange(n)]))
    for _ in range(20):
        perm = rng.permutation(n)
        a, b, c = np.split(perm, np.sort(rng.choice(np.arange(1, n), 2, replace=False)))
        sa = online_softmax_row(s, v, [a])
        sb = online_softmax_row(s, v, [b])
        sc = online_softmax_row(s, v, [c])
        for merged in (merge_states(merge_states(sa, sb), sc),
                       merge_states(sa, merge_states(sb, sc)),
                       merge_states(sc, merge_states(sb, sa))):
            mo, ml = finish(merged)
            np.testing.assert_allclose(mo, full_o, rtol=1e-13, atol=1e-13)
            assert abs(ml - full_l) < 1e-13 * max(1, abs(ml))


def test_two_block_statistics_example():
    g = json.load(open(os.path.join(GOLDEN, "two_block_statistics.json")))
    vals = np.array(g["values"])
    for case in g["cases"]:
        w = np.array(case["weights"], dtype=np.float64)
        s = np.log(w)
        exp = case["expected_num"] / case["expected_den"]
        # full definition: one query, two keys with bias ln(w), Q = 0
        q = np.zeros((1, 1, 2, 1))
        k = np.zeros((1, 1, 2, 1))
        v = np.zeros((1, 1, 2, 1))
        v[0, 0, :, 0] = vals
        bias = np.tile(s, (2, 1))[None, None]
        o, lse = sdpa_reference(q, k, v, bias, False)
        assert abs(o[0, 0, 0, 0] - exp) < 1e-15
        assert abs(lse[0, 0, 0] - math.log(3.0)) < 1e-15
        # block recurrence, one value per block, both orders
        for blocks in ([np.array([0]), np.array([1])], [np.array([1]), np.array([0])]):
            oi, _ = finish(online_softmax_row(s, vals[:, None], blocks))
            assert abs(oi[0] - exp) < 1e-15
        # per-block normalised outputs carry no weighting information
        per_block = [finish(online_softmax_row(s, vals[:, None], [np.array([j])]))[0][0]
                     for j in range(2)]
        assert per_block == g["per_block_normalised"]


def test_one_element_update_formulas():
    """The single-step update of the online softmax (running max m, normaliser l,
    value sum u; r = e^{m-m'}, l' = r l + p, u' = r u + p v with p = e^{s-m'}),
    applied one key at a time, reaches the full softmax. Page 'AI Infra 第5章图解',
    example 5-6; the widget's numbers are lost, so they are not pinned."""
    rng = _rng(5)
    s = rng.standard_normal(12) * 3
    s = np.append(s, math.log(4.0))          # a score of ln 4 ...
    vals = np.append(rng.standard_normal(12), 5.0)   # ... with value 5 (exercise 5-3)
    m, ell, u = -math.inf, 0.0, 0.0
    for sj, vj in zip(s, vals):
        m2 = max(m, sj)
        r = math.exp(m - m2)
        p = math.exp(sj - m2)
        ell = r * ell + p
        u = r * u + p * vj
        m = m2
    # full definition with Q = 0 and the scores carried by the bias
    n = len(s)
    bias = np.tile(s, (n, 1))[None, None]
    o, lse = sdpa_reference(np.zeros((1, 1, n, 1)), np.zeros((1, 1, n, 1)),
                            vals.reshape(1, 1, n, 1), bias, False)
    assert abs(o[0, 0, 0, 0] - u / ell) < 1e-13
    assert abs(lse[0, 0, 0] - (m + math.log(ell))) < 1e-13


# ---------------------------------------------------------------------------
# 4. closed forms and special cases
# ---------------------------------------------------------------------------

def test_q_zero_causal_is_cumulative_mean():
    rng = _rng(11)
    n, d, dv = 37, 8, 5
    v = rng.standard_normal((1, 2, n, dv))
    k = rng.standard_normal((1, 2, n, d))
    q = np.zeros((1, 2, n, d))
    o, lse = sdpa_reference(q, k, v, None, True)
    cm = np.cumsum(v, axis=2) / np.arange(1, n + 1)[None, None, :, None]
    np.testing.assert_allclose(o, cm, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, n + 1)), lse.shape),
                               rtol=1e-14)


def test_single_allowed_key_returns_that_value_exactly():
    rng = _rng(12)
    n, d, dv = 16, 8, 6
    q = rng.standard_normal((1, 1, n, d))
    k = rng.standard_normal((1, 1, n, d))
    v = rng.standard_normal((1, 1, n, dv))
    o, _ = sdpa_reference(q, k, v, None, True)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])          # causal row 0
    bias = np.full((1, 1, n, n), -np.inf)
    pick = rng.integers(0, n, size=n)
    bias[0, 0, np.arange(n), pick] = rng.standard_normal(n)
    o, lse = sdpa_reference(q, k, v, bias, False)
    assert np.array_equal(o[0, 0], v[0, 0, pick])


def test_constant_v():
    rng = _rng(13)
    n, d = 40, 16
    q = rng.standard_normal((2, 3, n, d)) * 3
    k = rng.standard_normal((2, 3, n, d)) * 3
    v = np.full((2, 3, n, 7), -2.75)
    o, _ = sdpa_reference(q, k, v, None, True)
    np.testing.assert_allclose(o, -2.75, rtol=1e-15)


def test_shift_invariance_of_bias_rows():
    rng = _rng(14)
    n, d, dv = 24, 8, 4
    q = rng.standard_normal((1, 1, n, d))
    k = rng.standard_normal((1, 1, n, d))
    v = rng.standard_normal((1, 1, n, dv))
    bias = rng.standard_normal((1, 1, n, n))
    c = rng.standard_normal(n) * 5
    o1, l1 = sdpa_reference(q, k, v, bias, True)
    o2, l2 = sdpa_reference(q, k, v, bias + c[None, None, :, None], True)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2 - l1, np.broadcast_to(c, l1.shape), rtol=1e-12, atol=1e-12)


def test_key_permutation_invariance_noncausal():
    rng = _rng(15)
    n, d, dv = 30, 8, 4
    q = rng.standard_normal((1, 1, n, d))
    k = rng.standard_normal((1, 1, n, d))
    v = rng.standard_normal((1, 1, n, dv))
    bias = rng.standard_normal((1, 1, n, n))
    perm = rng.permutation(n)
    o1, l1 = sdpa_reference(q, k, v, bias, False)
    o2, l2 = sdpa_reference(q, k[:, :, perm], v[:, :, perm], bias[:, :, :, perm], False)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-13)


def test_convexity_and_lse_bounds():
    rng = _rng(16)
    n, d, dv = 33, 16, 8
    q = rng.standard_normal((1, 1, n, d)) * 2
    k = rng.standard_normal((1, 1, n, d)) * 2
    v = rng.standard_normal((1, 1, n, dv))
    o, lse = sdpa_reference(q, k, v, None, True)
    s = _scores(q[0, 0], k[0, 0], None, True)
    for i in range(n):
        vi = v[0, 0, :i + 1]
        assert np.all(o[0, 0, i] >= vi.min(axis=0) - 1e-12)
        assert np.all(o[0, 0, i] <= vi.max(axis=0) + 1e-12)
        mx = s[i, :i + 1].max()
        assert mx - 1e-12 <= lse[0, 0, i] <= mx + math.log(i + 1) + 1e-12


def test_bias_broadcast_over_batch_and_heads():
    rng = _rng(17)
    B, H, n, d = 2, 3, 10, 4
    q = rng.standard_normal((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    v = rng.standard_normal((B, H, n, d))
    bias = rng.standard_normal((1, H, n, n))
    o, lse = sdpa_reference(q, k, v, bias, False)
    o2, lse2 = sdpa_reference(q, k, v, np.broadcast_to(bias, (B, H, n, n)).copy(), False)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_rows_sampler_matches_full():
    rng = _rng(18)
    B, H, n, d, dv = 2, 2, 50, 8, 16
    q = rng.standard_normal((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    v = rng.standard_normal((B, H, n, dv))
    bias = rng.standard_normal((1, H, n, n))
    o, lse = sdpa_reference(q, k, v, bias, True, row_chunk=7)
    rows = [0, 3, 17, 49]
    ro, rl = sdpa_reference_rows(q, k, v, bias, True, 1, 1, rows)
    np.testing.assert_allclose(ro, o[1, 1, rows], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(rl, lse[1, 1, rows], rtol=1e-14)


def test_empty_row_precondition_and_convention():
    q = np.zeros((1, 1, 3, 2))
    v = np.ones((1, 1, 3, 2))
    bias = np.zeros((1, 1, 3, 3))
    bias[0, 0, 1, :] = -np.inf
    with pytest.raises(EmptyRowError):
        sdpa_reference(q, q, v, bias, False)
    o, lse = sdpa_reference(q, q, v, bias, False, allow_empty_rows=True)
    assert np.all(o[0, 0, 1] == 0) and lse[0, 0, 1] == -np.inf
    assert np.all(o[0, 0, 0] == 1) and abs(lse[0, 0, 0] - math.log(3)) < 1e-15


def test_bf16_inputs_are_upcast_exactly():
    torch = pytest.importorskip("torch")
    x = torch.tensor([[[[1.0 + 2 ** -7, -3.0 - 2 ** -6]]]], dtype=torch.bfloat16)
    o, _ = sdpa_reference(x, x, x, None, False)
    assert o[0, 0, 0, 0] == 1.0 + 2 ** -7 and o[0, 0, 0, 1] == -3.0 - 2 ** -6


# ---------------------------------------------------------------------------
# N_q != N_k: the reading of the causal mask (queries aligned to the end of the keys)
# ---------------------------------------------------------------------------

def _rect(seed, nq, nk, d=5, dv=3, bias=False):
    rng = _rng(seed)
    q = rng.normal(size=(1, 2, nq, d))
    k = rng.normal(size=(1, 2, nk, d))
    v = rng.normal(size=(1, 2, nk, dv))
    c = rng.normal(size=(1, 2, nq, nk)) if bias else None
    return q, k, v, c


@pytest.mark.parametrize("nq,nk", [(3, 7), (7, 3), (1, 9), (5, 5)])
def test_rectangular_noncausal_brute_force(nq, nk):
    # without a mask every key is allowed: the plain definition, looped in pure Python
    q, k, v, c = _rect(40 + nq, nq, nk, bias=True)
    o, lse = sdpa_reference(q, k, v, c, False)
    for h in range(2):
        for i in range(nq):
            s = [math.fsum(q[0, h, i, t] * k[0, h, j, t] for t in range(5)) / math.sqrt(5) + c[0, h, i, j]
                 for j in range(nk)]
            w = [math.exp(x) for x in s]
            tot = math.fsum(w)
            want = [math.fsum(w[j] * v[0, h, j, t] for j in range(nk)) / tot for t in range(3)]
            np.testing.assert_allclose(o[0, h, i], want, rtol=1e-13, atol=1e-14)
            assert abs(lse[0, h, i] - math.log(tot)) < 1e-12


def test_single_query_row_sees_every_key():
    # one query row against N_k keys (decode): the causal mask forbids nothing
    q, k, v, c = _rect(50, 1, 12, bias=True)
    oc, lc = sdpa_reference(q, k, v, c, True)
    on, ln = sdpa_reference(q, k, v, c, False)
    np.testing.assert_array_equal(oc, on)
    np.testing.assert_array_equal(lc, ln)


@pytest.mark.parametrize("nq", [1, 4, 11])
def test_query_rows_are_the_last_positions_of_the_sequence(nq):
    # N_q rows against N_k keys under the causal mask equal the last N_q rows of the
    # square causal problem whose queries end with them
    nk = 11
    rng = _rng(60 + nq)
    qf = rng.normal(size=(1, 2, nk, 4))
    k = rng.normal(size=(1, 2, nk, 4))
    v = rng.normal(size=(1, 2, nk, 3))
    cf = rng.normal(size=(1, 2, nk, nk))
    of, lf = sdpa_reference(qf, k, v, cf, True)
    o, lse = sdpa_reference(qf[:, :, nk - nq:], k, v, cf[:, :, nk - nq:], True)
    np.testing.assert_allclose(o, of[:, :, nk - nq:], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse, lf[:, :, nk - nq:], rtol=1e-14, atol=1e-15)


def test_more_query_rows_than_keys():
    # N_q > N_k under the causal mask: the first N_q - N_k rows see no key (precondition
    # violated: the oracle raises, or returns the O = 0, lse = -inf convention); the
    # others are the square problem
    q, k, v, _ = _rect(70, 9, 4)
    with pytest.raises(EmptyRowError):
        sdpa_reference(q, k, v, None, True)
    o, lse = sdpa_reference(q, k, v, None, True, allow_empty_rows=True)
    assert (o[:, :, :5] == 0).all() and np.isneginf(lse[:, :, :5]).all()
    o2, l2 = sdpa_reference(q[:, :, 5:], k, v, None, True)
    np.testing.assert_array_equal(o[:, :, 5:], o2)
    np.testing.assert_array_equal(lse[:, :, 5:], l2)
