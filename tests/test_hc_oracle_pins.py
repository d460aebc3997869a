"""Pins of the Hyper-Connection mixer oracle (P1 s10) against what the page and
the mathematics fix: Sinkhorn output is doubly stochastic and equals the
Sinkhorn-Knopp scaling limit computed another way; rank-one entries give the
uniform matrix; a hand-computed first iteration; permutation equivariance;
closed forms of the logistic gates; the stream mixes on special cases,
including which index of the coupling matrix gathers (a 3-cycle)."""
import math

import numpy as np
import pytest

import oracle as O

RNG = np.random.default_rng(20260)


def test_sinkhorn_is_doubly_stochastic():
    m = RNG.standard_normal((64, 4, 4))
    c = O.sinkhorn(m)
    assert np.all(c > 0)
    # the last step normalises columns: each sums to s / (s + eps)
    assert np.allclose(c.sum(-2), 1.0, atol=2e-6)
    assert np.allclose(c.sum(-1), 1.0, atol=5e-4)   # 20 iterations from N(0, 1) entries


def _sinkhorn_knopp_limit(a, iters=20000):
    """Scaling vectors r, s with diag(r) A diag(s) doubly stochastic, by the
    fixed point r = 1 / (A s), s = 1 / (A^T r) (no matrix normalisation)."""
    s = np.ones(a.shape[-1])
    for _ in range(iters):
        r = 1.0 / (a @ s)
        s = 1.0 / (a.T @ r)
    return r[:, None] * a * s[None, :]


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_sinkhorn_reaches_the_scaling_limit(seed):
    m = np.random.default_rng(seed).standard_normal((4, 4)) * 0.5
    ref = _sinkhorn_knopp_limit(np.exp(m))
    got = O.sinkhorn(m, iters=200, eps=0.0)
    assert np.allclose(got, ref, atol=1e-12)
    # 20 iterations at this conditioning are already within 1e-6 of the limit
    assert np.allclose(O.sinkhorn(m, iters=20, eps=0.0), ref, atol=1e-6)


def test_rank_one_entries_give_the_uniform_matrix():
    a, b = RNG.standard_normal(4), RNG.standard_normal(4)
    m = a[:, None] + b[None, :]
    assert np.allclose(O.sinkhorn(m, eps=0.0), 0.25, atol=1e-15)


def test_first_iteration_by_hand():
    # row 0 = (ln 3, 0, 0, 0), other rows zero: the row softmax gives row 0 =
    # (1/2, 1/6, 1/6, 1/6) and 1/4 elsewhere; column 0 sums to 5/4, the others
    # to 11/12, so C[0][0] = 0.4, C[0][1] = 2/11, C[1][0] = 0.2, C[1][1] = 3/11
    m = np.zeros((4, 4))
    m[0, 0] = math.log(3.0)
    c = O.sinkhorn(m, iters=1, eps=0.0)
    assert c[0, 0] == pytest.approx(0.4, abs=1e-15)
    assert c[0, 1] == pytest.approx(2.0 / 11.0, abs=1e-15)
    assert c[1, 0] == pytest.approx(0.2, abs=1e-15)
    assert c[1, 1] == pytest.approx(3.0 / 11.0, abs=1e-15)


def test_sinkhorn_is_permutation_equivariant():
    m = RNG.standard_normal((4, 4))
    p, q = RNG.permutation(4), RNG.permutation(4)
    assert np.allclose(O.sinkhorn(m[p][:, q]), O.sinkhorn(m)[p][:, q], atol=1e-14)


def test_gates_are_logistic():
    mix = np.zeros(24)
    mix[1], mix[5] = math.log(3.0), -math.log(3.0)
    pre, post, comb = O.hc_split(mix)
    assert pre[0] == 0.5 and pre[1] == pytest.approx(0.75, abs=1e-15)
    assert post[1] == pytest.approx(0.25, abs=1e-15)
    x = RNG.standard_normal(8)
    assert np.allclose(O.sigmoid(x) + O.sigmoid(-x), 1.0, atol=1e-15)
    assert comb.shape == (4, 4)


def test_pre_mix_special_cases():
    h = RNG.standard_normal((4, 32))
    # gates saturated to one-hot: the block input is that stream
    mix = np.full(24, -60.0)
    mix[2] = 60.0
    pre, _, _ = O.hc_split(mix)
    assert np.allclose(O.hc_pre(pre, h), h[2], atol=1e-12)
    # equal streams: the input is the gate sum times the stream
    hs = np.repeat(h[:1], 4, axis=0)
    pre = np.array([0.1, 0.2, 0.3, 0.9])
    assert np.allclose(O.hc_pre(pre, hs), 1.5 * h[0], atol=1e-14)


def test_post_mix_gathers_along_rows():
    h = RNG.standard_normal((4, 16))
    y = RNG.standard_normal(16)
    # a 3-cycle: C ~ P with P[0][1] = P[1][2] = P[2][0] = P[3][3] = 1
    mix = np.zeros(24)
    cm = np.full((4, 4), -30.0)
    for j, i in ((0, 1), (1, 2), (2, 0), (3, 3)):
        cm[j, i] = 30.0
    mix[8:] = cm.reshape(-1)
    mix[4:8] = [60.0, -60.0, 60.0, -60.0]   # post gates 1, 0, 1, 0
    _, post, comb = O.hc_split(mix)
    out = O.hc_post(post, comb, h, y)
    # (C's entries are 1 - 1e-6 there: the eps of each normalisation)
    assert np.allclose(out[0], h[1] + y, atol=1e-5)
    assert np.allclose(out[1], h[2], atol=1e-5)
    assert np.allclose(out[2], h[0] + y, atol=1e-5)
    assert np.allclose(out[3], h[3], atol=1e-5)
    # equal streams and a doubly stochastic C: every stream becomes h + post_j y
    hs = np.repeat(h[:1], 4, axis=0)
    pre, post, comb = O.hc_split(RNG.standard_normal(24))
    out = O.hc_post(post, comb, hs, y)
    for j in range(4):
        assert np.allclose(out[j], h[0] + post[j] * y, atol=5e-4 * np.abs(h[0]).max())
