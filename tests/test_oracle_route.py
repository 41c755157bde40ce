"""Pins of the oracle's routing against facts that do not come from the oracle itself:
brute-force enumeration, library routines (scipy softmax / expit), invariants of the method
and hand-worked examples.

Routing as defined by the TileOPs "MoE" page (FusedTopKFwd and FusedMoEFwd attributes:
top_k, scoring_func, renormalize, num_expert_group, topk_group, routed_scaling_factor,
correction_bias)."""
import itertools

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _keys(g, scoring, bias):
    """Selection keys restated from the definition (softmax: logits; sigmoid: f32 score + f32
    bias) -- used only to drive the brute-force enumeration below."""
    if scoring == "softmax":
        return g.astype(np.float32)
    s32 = expit(g.astype(np.float64)).astype(np.float32)
    b = np.zeros_like(s32) if bias is None else bias.astype(np.float32)
    return (s32 + b).astype(np.float32)


def _brute_force_ids(key, k, n_group, topk_group):
    """Enumerate every choice of topk_group groups; the kept set is the one whose sorted group
    scores are lexicographically largest (ties: lower group indices), then a full stable sort of
    the eligible experts by (-key, index)."""
    E = key.size
    gs = E // n_group
    if n_group > 1:
        gscore = []
        for g in range(n_group):
            kk = np.sort(key[g * gs:(g + 1) * gs])[::-1]
            gscore.append(np.float32(kk[0] + kk[1]) if gs > 1 else kk[0])
        best = None
        for subset in itertools.combinations(range(n_group), topk_group):
            # rank of a subset: its group scores in descending order, then its indices ascending
            rank = (sorted([gscore[g] for g in subset], reverse=True),
                    [-g for g in sorted(subset, key=lambda g: (-gscore[g], g))])
            if best is None or rank > best[0]:
                best = (rank, subset)
        allowed = np.zeros(E, bool)
        for g in best[1]:
            allowed[g * gs:(g + 1) * gs] = True
    else:
        allowed = np.ones(E, bool)
    idx = np.arange(E)[allowed]
    order = np.lexsort((idx, -key[allowed].astype(np.float64)))
    return idx[order][:k]


CASES = [
    # (E, k, scoring, bias, n_group, topk_group, renorm, rsf)
    (8, 2, "softmax", False, 1, 1, True, 1.0),
    (16, 4, "softmax", False, 1, 1, False, 1.0),
    (32, 8, "sigmoid", True, 1, 1, True, 2.827),
    (32, 8, "sigmoid", True, 8, 4, True, 2.5),
    (24, 3, "sigmoid", True, 6, 2, True, 1.5),
    (12, 5, "sigmoid", False, 4, 3, False, 1.0),
    (16, 4, "sigmoid", True, 16, 5, True, 1.0),   # groups of one expert
]


@pytest.mark.parametrize("E,k,scoring,use_bias,n_group,topk_group,renorm,rsf", CASES)
def test_route_matches_brute_force(E, k, scoring, use_bias, n_group, topk_group, renorm, rsf):
    r = _rng(E * 100 + k)
    T = 200
    g = r.standard_normal((T, E)).astype(np.float32)
    bias = (0.1 * r.standard_normal(E)).astype(np.float32) if use_bias else None
    ids, w = oracle.route(g, bias, k, scoring, renorm, n_group, topk_group, rsf)
    for t in range(T):
        key = _keys(g[t], scoring, bias)
        expect = _brute_force_ids(key, k, n_group, topk_group)
        assert list(ids[t]) == list(expect), (t, ids[t], expect)


@pytest.mark.parametrize("E,k,scoring,use_bias,n_group,topk_group,renorm,rsf", CASES)
def test_route_invariants(E, k, scoring, use_bias, n_group, topk_group, renorm, rsf):
    r = _rng(E * 7 + k)
    T = 300
    g = r.standard_normal((T, E)).astype(np.float32)
    bias = (0.1 * r.standard_normal(E)).astype(np.float32) if use_bias else None
    ids, w = oracle.route(g, bias, k, scoring, renorm, n_group, topk_group, rsf)
    gs = E // n_group
    for t in range(T):
        assert len(set(ids[t].tolist())) == k                      # k distinct experts
        assert ids[t].min() >= 0 and ids[t].max() < E
        assert len(set((ids[t] // gs).tolist())) <= topk_group       # confined to kept groups
        key = _keys(g[t], scoring, bias)[ids[t]]
        assert np.all(key[:-1] >= key[1:])                           # descending key order
        assert np.all(w[t] > 0)
        if renorm:
            assert abs(float(np.sum(w[t], dtype=np.float64)) / rsf - 1.0) <= 1e-6
    if scoring == "softmax":
        assert np.all(w[:, :-1] >= w[:, 1:])                         # softmax weights descend


def test_softmax_full_k_is_softmax():
    """k = E, no renormalize: the weights are the row softmax (library routine), listed in
    descending-logit order."""
    r = _rng(1)
    g = r.standard_normal((50, 16)).astype(np.float32)
    ids, w = oracle.route(g, None, 16, "softmax", False)
    ref = softmax(g.astype(np.float64), axis=1)
    for t in range(50):
        assert np.allclose(w[t], ref[t, ids[t]], rtol=0, atol=1e-7)
        assert list(ids[t]) == list(np.argsort(-g[t], kind="stable"))


def test_softmax_renormalized_is_softmax_of_selected():
    """Renormalized softmax top-k = softmax over the selected logits, times rsf."""
    r = _rng(2)
    g = r.standard_normal((80, 64)).astype(np.float32)
    ids, w = oracle.route(g, None, 6, "softmax", True, rsf=1.7)
    for t in range(80):
        ref = softmax(g[t, ids[t]].astype(np.float64)) * 1.7
        assert np.allclose(w[t], ref, rtol=0, atol=2e-7)


def test_sigmoid_weights_use_unbiased_scores():
    """The correction bias steers the choice only: weights are expit(logit) of the chosen
    experts, renormalized and scaled."""
    r = _rng(3)
    g = r.standard_normal((60, 32)).astype(np.float32)
    bias = (0.5 * r.standard_normal(32)).astype(np.float32)
    ids, w = oracle.route(g, bias, 8, "sigmoid", True, rsf=2.5)
    for t in range(60):
        s = expit(g[t, ids[t]].astype(np.float64))
        assert np.allclose(w[t], s / s.sum() * 2.5, rtol=0, atol=1e-6)
    ids0, _ = oracle.route(g, None, 8, "sigmoid", True)
    assert not np.array_equal(ids0, ids)        # a bias this large changes some choices


def test_sigmoid_without_bias_is_topk_of_logits():
    """sigmoid is increasing, so without bias the choice is the top-k of the logits (unless
    f32 rounding of the score ties two experts; N(0,1) logits are far from saturation)."""
    r = _rng(4)
    g = r.standard_normal((100, 64)).astype(np.float32)
    ids, _ = oracle.route(g, None, 8, "sigmoid", False)
    for t in range(100):
        assert list(ids[t]) == list(np.argsort(-g[t], kind="stable")[:8])


def test_sigmoid_no_renorm_weight_is_rsf_times_score():
    r = _rng(5)
    g = r.standard_normal((20, 16)).astype(np.float32)
    ids, w = oracle.route(g, None, 4, "sigmoid", False, rsf=2.0)
    assert np.allclose(w, 2.0 * expit(np.take_along_axis(g.astype(np.float64), ids, 1)),
                       rtol=0, atol=1e-7)


def test_grouping_reduces_to_plain_topk():
    """num_expert_group = 1, or topk_group = num_expert_group, is plain top-k."""
    r = _rng(6)
    g = r.standard_normal((100, 32)).astype(np.float32)
    bias = (0.1 * r.standard_normal(32)).astype(np.float32)
    a = oracle.route(g, bias, 8, "sigmoid", True, 1, 1, 2.5)
    b = oracle.route(g, bias, 8, "sigmoid", True, 8, 8, 2.5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_hand_worked_softmax():
    g = np.array([[1.0, 3.0, 2.0, 0.0]], np.float32)
    ids, w = oracle.route(g, None, 2, "softmax", True)
    assert list(ids[0]) == [1, 2]
    e = np.exp(1.0)
    assert np.allclose(w[0], [e / (e + 1), 1 / (e + 1)], rtol=0, atol=1e-7)


def test_hand_worked_ties_go_to_lower_index():
    g = np.zeros((1, 6), np.float32)
    ids, w = oracle.route(g, None, 3, "softmax", True)
    assert list(ids[0]) == [0, 1, 2]
    assert np.allclose(w[0], 1 / 3, atol=1e-7)
    # group ties: 3 groups of 2 with equal group scores -> the two lower groups are kept
    ids, _ = oracle.route(g, None, 4, "sigmoid", True, 3, 2)
    assert sorted(ids[0].tolist()) == [0, 1, 2, 3]


def test_hand_worked_group_score_is_top2_sum():
    """Group 0 holds the single largest key but group 1 has the larger top-2 sum, so with
    topk_group = 1 only group 1's experts can be chosen."""
    # keys via sigmoid of these logits (4 groups of 3)
    g = np.array([[4.0, -3.0, -3.0,    2.0, 2.0, -3.0,    -1.0, -1.0, -1.0,   0.0, -3.0, -3.0]],
                 np.float32)
    ids, _ = oracle.route(g, None, 2, "sigmoid", True, 4, 1)
    assert sorted(ids[0].tolist()) == [3, 4]
    ids, _ = oracle.route(g, None, 2, "sigmoid", True, 4, 2)
    assert sorted(ids[0].tolist()) == [0, 3]      # groups 0 and 1 kept; best keys 4.0, then 2.0


def test_rejects_unsupported():
    g = np.zeros((2, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.route(g, None, 9)                       # k > E
    with pytest.raises(ValueError):
        oracle.route(g, None, 2, "sigmoid", True, 3, 1)  # E not divisible by groups
    with pytest.raises(ValueError):
        oracle.route(g, None, 5, "sigmoid", True, 4, 2)  # k > experts in kept groups
