"""Pins of the grouped sigmoid router oracle (oracle.route_grouped) against
things other than itself: a sort-based brute force in numpy (stable sorts
instead of repeated arg-max), the plain softmax router it must agree with
when there is one group and no bias (sigmoid and softmax order experts the
same way), the group restriction, bias that moves the choice but never the
weights, exact scaling by a power of two, and tie-breaking.  CPU only.
"""
import numpy as np
import pytest

import oracle


def sigmoid32(l):
    l = np.asarray(l, np.float32)
    return (np.float32(1) / (np.float32(1) + np.exp(-l))).astype(np.float32)


def brute_force(logits, k, n_group, topk_group, bias=None, scale=1.0):
    """Stable sorts over (score, id): group scores from the two largest of a
    sorted group, groups and experts taken from lexicographic orders."""
    T, E = logits.shape
    G = E // n_group
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    for t in range(T):
        s = sigmoid32(logits[t]).astype(np.float64)
        c = (sigmoid32(logits[t]) + (np.zeros(E, np.float32) if bias is None
                                     else np.asarray(bias, np.float32))).astype(np.float64)
        gsc = []
        for g in range(n_group):
            top = np.sort(c[g * G:(g + 1) * G])[::-1]
            gsc.append(top[0] + (top[1] if G > 1 else 0.0))
        order_g = sorted(range(n_group), key=lambda g: (-gsc[g], g))
        kept = set(order_g[:topk_group])
        cand = [e for e in range(E) if e // G in kept]
        order_e = sorted(cand, key=lambda e: (-c[e], e))
        ids[t] = order_e[:k]
        w[t] = s[ids[t]] / s[ids[t]].sum() * scale
    return ids, w


@pytest.mark.parametrize("E,n_group,topk_group,k", [
    (256, 8, 4, 8), (64, 4, 2, 6), (32, 32, 8, 8), (16, 2, 1, 4), (60, 6, 3, 5), (8, 1, 1, 2),
])
def test_matches_sort_based_brute_force(E, n_group, topk_group, k):
    rng = np.random.default_rng(E + n_group + k)
    lg = rng.standard_normal((24, E)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.05).astype(np.float32)
    for b in (None, bias):
        ids, w = oracle.route_grouped(lg, k, n_group, topk_group, bias=b, scale=2.5)
        rid, rw = brute_force(lg, k, n_group, topk_group, bias=b, scale=2.5)
        assert np.array_equal(ids, rid)
        np.testing.assert_allclose(w, rw, rtol=2e-6, atol=0)


def test_one_group_no_bias_is_the_softmax_routers_choice():
    """Sigmoid and softmax are both increasing in the logit, so with a single
    group and no bias the chosen ids (and their order) are the softmax
    router's; the weights are the normalised sigmoids."""
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((50, 128)).astype(np.float32)
    ids, w = oracle.route_grouped(lg, 8, 1, 1)
    sid, _ = oracle.route_topk(lg, 8)
    assert np.array_equal(ids, sid)
    s = sigmoid32(lg).astype(np.float64)
    ref = np.take_along_axis(s, ids, 1)
    np.testing.assert_allclose(w, ref / ref.sum(1, keepdims=True), rtol=2e-6)


def test_choices_stay_inside_the_best_groups():
    rng = np.random.default_rng(2)
    E, n_group, tg, k = 256, 8, 4, 8
    lg = rng.standard_normal((40, E)).astype(np.float32)
    ids, _ = oracle.route_grouped(lg, k, n_group, tg)
    G = E // n_group
    for t in range(40):
        c = sigmoid32(lg[t]).astype(np.float64)
        gs = np.array([np.sort(c[g * G:(g + 1) * G])[-2:].sum() for g in range(n_group)])
        best = set(np.argsort(-gs, kind="stable")[:tg].tolist())
        assert {int(e) // G for e in ids[t]} <= best
        assert len(set(ids[t].tolist())) == k


def test_bias_moves_the_choice_but_not_the_weights():
    """A large bias on expert 5 forces it in (it is chosen first); the
    weights are still the chosen experts' normalised sigmoids, bias-free."""
    rng = np.random.default_rng(3)
    E = 64
    lg = rng.standard_normal((10, E)).astype(np.float32)
    bias = np.zeros(E, np.float32)
    bias[5] = 10.0
    ids, w = oracle.route_grouped(lg, 4, 4, 2, bias=bias)
    assert np.all(ids[:, 0] == 5)
    s = sigmoid32(lg).astype(np.float64)
    ref = np.take_along_axis(s, ids, 1)
    np.testing.assert_allclose(w, ref / ref.sum(1, keepdims=True), rtol=2e-6)


def test_power_of_two_scale_is_exact():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((16, 256)).astype(np.float32)
    ids1, w1 = oracle.route_grouped(lg, 8, 8, 4, scale=1.0)
    ids2, w2 = oracle.route_grouped(lg, 8, 8, 4, scale=4.0)
    assert np.array_equal(ids1, ids2)
    assert np.array_equal(w2, w1 * np.float32(4.0))


def test_ties_go_to_the_lower_id_and_group():
    """Equal logits everywhere: every group ties, every expert ties; the
    lowest groups and the lowest ids win, in ascending order, with equal
    weights."""
    E, n_group, tg, k = 32, 4, 2, 5
    lg = np.zeros((2, E), np.float32)
    ids, w = oracle.route_grouped(lg, k, n_group, tg)
    assert ids.tolist() == [[0, 1, 2, 3, 4]] * 2
    assert np.all(w == np.float32(0.2))
    lg[:, 8:16] = 1.0                    # group 1 now best, group 0 next
    ids, _ = oracle.route_grouped(lg, k, n_group, tg)
    assert ids.tolist() == [[8, 9, 10, 11, 12]] * 2
