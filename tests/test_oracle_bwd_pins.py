"""Pins for the gradient oracle (oracle/backward.py).

The pages print no gradient formulas, so each pin reaches the gradients by another
route: central finite differences of the (separately pinned) forward oracle, automatic
differentiation of a plain softmax composition, closed forms of special cases, and
invariants that hold for any inputs. A dropped term of the softmax Jacobian, a wrong
scale, a transposed product or a mask applied in the wrong direction fails one of them.
"""

import math

import numpy as np
import pytest

from oracle import sdpa_backward_reference, sdpa_backward_reference_sampled, sdpa_reference


def _case(seed, B=1, H=2, N=6, d=4, dv=3, bias=False, causal=False, masked_frac=0.25):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(B, H, N, d))
    k = rng.normal(size=(B, H, N, d))
    v = rng.normal(size=(B, H, N, dv))
    do = rng.normal(size=(B, H, N, dv))
    c = None
    if bias:
        c = rng.normal(size=(1, H, N, N))
        kill = rng.random((1, H, N, N)) < masked_frac
        kill[..., np.arange(N), np.arange(N)] = False  # every row keeps a key
        c[kill] = -np.inf
    return q, k, v, do, c


def _loss(q, k, v, c, causal, g):
    o, _ = sdpa_reference(q, k, v, c, causal)
    return float((o * g).sum())


@pytest.mark.parametrize("seed,bias,causal,d,dv", [
    (1, False, False, 4, 3), (2, False, True, 4, 3), (3, True, False, 5, 2), (4, True, True, 3, 6),
])
def test_central_differences_of_the_forward(seed, bias, causal, d, dv):
    q, k, v, do, c = _case(seed, bias=bias, causal=causal, d=d, dv=dv)
    dq, dk, dvv = sdpa_backward_reference(q, k, v, do, c, causal)
    h = 1e-5
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dvv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            lp = _loss(*(xp if n == name else args[n] for n in "qkv"), c, causal, do)
            lm = _loss(*(xm if n == name else args[n] for n in "qkv"), c, causal, do)
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8, err_msg=name)


def test_automatic_differentiation_of_plain_softmax():
    torch = pytest.importorskip("torch")
    q, k, v, do, c = _case(7, B=2, H=3, N=37, d=16, dv=8, bias=True, causal=True)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = tq @ tk.transpose(-1, -2) / math.sqrt(16) + torch.tensor(c)
    s = s.masked_fill(torch.ones(37, 37, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    o.backward(torch.tensor(do))
    dq, dk, dvv = sdpa_backward_reference(q, k, v, do, c, True)
    for ours, ref in ((dq, tq.grad), (dk, tk.grad), (dvv, tv.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_single_allowed_key_rows():
    # every row may use one key only: P is 1 there, so dS = 0 (no gradient reaches Q or
    # K) and dV of key j is the sum of dO over the rows that pick j
    rng = np.random.default_rng(11)
    N, d, dv = 9, 4, 3
    q, k, v, do, _ = _case(11, B=1, H=1, N=N, d=d, dv=dv)
    pick = rng.integers(0, N, size=N)
    c = np.full((1, 1, N, N), -np.inf)
    c[0, 0, np.arange(N), pick] = rng.normal(size=N)
    dq, dk, dvv = sdpa_backward_reference(q, k, v, do, c, False)
    assert (dq == 0).all() and (dk == 0).all()
    want = np.zeros((N, dv))
    for i in range(N):
        want[pick[i]] += do[0, 0, i]
    np.testing.assert_array_equal(dvv[0, 0], want)


def test_constant_v_gives_no_score_gradient():
    q, k, _, do, c = _case(12, N=8, bias=True, causal=True)
    v = np.full((1, 2, 8, 3), -0.75)
    dq, dk, _ = sdpa_backward_reference(q, k, v, do, c, True)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14


def test_zero_queries_causal_closed_form():
    # Q = 0, causal: P_ij = 1/(i+1) for j <= i, so dV_j = sum_{i >= j} dO_i / (i+1)
    _, k, v, do, _ = _case(13, N=10)
    q = np.zeros((1, 2, 10, 4))
    _, _, dvv = sdpa_backward_reference(q, k, v, do, None, True)
    w = do / np.arange(1, 11)[None, None, :, None]
    want = np.flip(np.cumsum(np.flip(w, axis=2), axis=2), axis=2)
    np.testing.assert_allclose(dvv, want, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_sums(causal):
    # rows of P sum to one: the dV rows add up to the dO rows; the rows of dS sum to
    # zero: the dK rows add up to zero (a shift of every key moves no probability)
    q, k, v, do, c = _case(14, B=2, H=2, N=23, d=8, dv=5, bias=True, causal=causal)
    _, dk, dvv = sdpa_backward_reference(q, k, v, do, c, causal)
    np.testing.assert_allclose(dvv.sum(axis=2), do.sum(axis=2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)


def test_linear_in_the_upstream_gradient():
    q, k, v, do, c = _case(15, N=12, bias=True, causal=True)
    do2 = np.random.default_rng(16).normal(size=do.shape)
    g1 = sdpa_backward_reference(q, k, v, do, c, True)
    g2 = sdpa_backward_reference(q, k, v, do2, c, True)
    g3 = sdpa_backward_reference(q, k, v, 2 * do - do2, c, True)
    for a, b_, s in zip(g1, g2, g3):
        np.testing.assert_allclose(s, 2 * a - b_, rtol=1e-12, atol=1e-12)


def test_sampled_and_chunked_match_full():
    q, k, v, do, c = _case(17, B=2, H=2, N=50, d=8, dv=6, bias=True, causal=True)
    full = sdpa_backward_reference(q, k, v, do, c, True)
    chunked = sdpa_backward_reference(q, k, v, do, c, True, row_chunk=7)
    for a, b_ in zip(full, chunked):
        np.testing.assert_allclose(a, b_, rtol=1e-13, atol=1e-14)
    rows, keys = [0, 17, 49], [0, 3, 31, 49]
    dq, dk, dvv = sdpa_backward_reference_sampled(q, k, v, do, c, True, 1, 0, rows, keys, row_chunk=9)
    np.testing.assert_allclose(dq, full[0][1, 0, rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dk, full[1][1, 0, keys], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dvv, full[2][1, 0, keys], rtol=1e-13, atol=1e-14)


def test_error_scales_sampled_match_full_and_bound_terms():
    # the tolerance scales: the sampled variant equals the full one, and each scale is
    # at least the root-sum-square of the plain terms of its gradient
    q, k, v, do, c = _case(18, B=1, H=2, N=40, d=8, dv=6, bias=True, causal=True)
    dq, dk, dvv, (sq, sk, sv) = sdpa_backward_reference(q, k, v, do, c, True, with_scales=True)
    rows, keys = [0, 7, 39], [0, 13, 39]
    res = sdpa_backward_reference_sampled(q, k, v, do, c, True, 0, 1, rows, keys, row_chunk=11,
                                          with_scales=True)
    np.testing.assert_allclose(res[3][0], sq[0, 1, rows], rtol=1e-12)
    np.testing.assert_allclose(res[3][1], sk[0, 1, keys], rtol=1e-12)
    np.testing.assert_allclose(res[3][2], sv[0, 1, keys], rtol=1e-12)
    assert (sq >= 0).all() and (sk >= 0).all() and (sv >= 0).all()
    # |dV_j| <= sum_i P_ij |dO_i| <= sqrt(n) * sv_j (Cauchy-Schwarz), with n = 40 rows
    assert (np.abs(dvv) <= math.sqrt(40) * sv + 1e-12).all()
