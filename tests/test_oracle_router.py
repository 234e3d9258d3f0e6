"""Pins of the oracle's router (logits, top-k, weights) and grouping."""
import numpy as np
import pytest
import scipy.special

from oracle import moe as om

RNG = np.random.default_rng(77)


def _router(E=16, H=64, T=5):
    x = RNG.standard_normal((T, H)).astype(np.float32)
    wr = (RNG.standard_normal((E, H)) * 0.02).astype(np.float32)
    return x, wr


def test_logits_are_exact_fp64_products():
    """Each fp32 x fp32 product is exact in fp64; a sum of such products over
    a power-of-two-scaled integer grid is exact, so the logit equals the
    integer dot product computed in Python integers."""
    H, E = 64, 8
    xi = RNG.integers(-2**11, 2**11, (3, H))
    wi = RNG.integers(-2**11, 2**11, (E, H))
    x = (xi * 2.0 ** -9).astype(np.float32)
    wr = (wi * 2.0 ** -13).astype(np.float32)
    lg = om.router_logits(x, wr)
    for t in range(3):
        for e in range(E):
            exact = sum(int(a) * int(b) for a, b in zip(xi[t], wi[e])) * 2.0 ** -22
            assert lg[t, e] == exact


def test_bias_added_and_zero_input():
    x, wr = _router()
    b = RNG.standard_normal(16).astype(np.float32)
    lg0 = om.router_logits(np.zeros_like(x), wr, b)
    assert np.array_equal(lg0, np.broadcast_to(b.astype(np.float64), lg0.shape))
    lg = om.router_logits(x, wr, b)
    assert np.allclose(lg - om.router_logits(x, wr), b[None, :], rtol=0, atol=1e-12)


def test_k1_is_argmax():
    x, wr = _router()
    lg = om.router_logits(x, wr)
    ids, w, _ = om.top_k(lg, 1)
    assert np.array_equal(ids[:, 0], np.argmax(lg, axis=1))
    assert np.all(w == 1.0)


def test_k_equals_E_is_full_softmax():
    x, wr = _router(E=12)
    lg = om.router_logits(x, wr)
    ids, w, _ = om.top_k(lg, 12)
    sm = scipy.special.softmax(lg, axis=1)
    for t in range(lg.shape[0]):
        assert sorted(ids[t]) == list(range(12))
        assert np.all(np.diff(lg[t, ids[t]]) <= 0)
        assert np.allclose(w[t], sm[t, ids[t]], rtol=1e-13, atol=0)


def test_softmax_then_renormalise_equals_selected_softmax():
    x, wr = _router(E=32)
    lg = om.router_logits(x, wr)
    ids, w, _ = om.top_k(lg, 4)
    sm = scipy.special.softmax(lg, axis=1)
    for t in range(lg.shape[0]):
        p = sm[t, ids[t]]
        assert np.allclose(w[t], p / p.sum(), rtol=1e-13, atol=0)
        assert abs(w[t].sum() - 1.0) < 1e-12


def test_ties_break_to_lower_index():
    x, wr = _router(E=16)
    wr[9] = wr[3]          # experts 3 and 9 get identical logits
    wr[12] = wr[3]
    lg = om.router_logits(x, wr)
    ids, w, gap = om.top_k(lg, 16)
    for t in range(lg.shape[0]):
        pos = {int(e): i for i, e in enumerate(ids[t])}
        assert pos[3] < pos[9] < pos[12]
        assert pos[9] == pos[3] + 1 and pos[12] == pos[9] + 1
        assert w[t, pos[3]] == w[t, pos[9]] == w[t, pos[12]]
    # all-equal logits: the first k indices, equal weights
    ids, w, gap = om.top_k(np.zeros((2, 10)), 4)
    assert np.array_equal(ids, [[0, 1, 2, 3]] * 2)
    assert np.allclose(w, 0.25) and np.all(gap == 0)


def test_permuting_experts_permutes_ids():
    x, wr = _router(E=24)
    perm = RNG.permutation(24)
    lg = om.router_logits(x, wr)
    ids, w, _ = om.top_k(lg, 5)
    ids_p, w_p, _ = om.top_k(om.router_logits(x, wr[perm]), 5)
    inv = np.argsort(perm)
    assert np.array_equal(perm[ids_p], ids)
    assert np.array_equal(w_p, w)
    assert inv is not None


def test_gap_is_kth_minus_next():
    lg = np.array([[3.0, 1.0, 2.0, 0.5, 2.5]])
    ids, w, gap = om.top_k(lg, 2)
    assert list(ids[0]) == [0, 4]
    assert gap[0] == 0.5
    e = np.exp([0.0, -0.5])
    assert np.allclose(w[0], e / e.sum(), rtol=1e-15)


@pytest.mark.parametrize("T,k,E", [(1, 2, 16), (4, 8, 256), (64, 8, 256), (7, 3, 5)])
def test_grouping_matches_stable_argsort(T, k, E):
    ids = np.stack([RNG.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    cnt, off, pairs, active = om.group_by_expert(ids, E)
    flat = ids.reshape(-1)
    assert np.array_equal(cnt, np.bincount(flat, minlength=E))
    assert np.array_equal(pairs, np.argsort(flat, kind="stable"))
    assert off[0] == 0 and off[-1] == T * k and np.array_equal(np.diff(off), cnt)
    assert np.array_equal(active, np.unique(flat))
