"""Pins of the oracle's router (sigmoid, biased top-4, weight normalisation).

Each test checks the oracle against something other than itself: the guide's
illustrative token, closed forms, brute force over every 4-subset, library
routines and invariants.  CPU only.
"""

import json
import math
import os
from itertools import combinations

import numpy as np
import pytest
import scipy.special
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _logit(p):
    return np.log(p) - np.log1p(-p)


def _illustrative():
    with open(os.path.join(GOLDEN, "illustrative_token.json")) as f:
        fx = json.load(f)
    E = oracle.EXPERTS
    s = np.empty(E)
    b = np.zeros(E)
    others = [e for e in range(E) if e >= 5]
    s[others] = np.linspace(fx["others"]["s_from"], fx["others"]["s_to"], len(others))
    names = {}
    for name, v in fx["candidates"].items():
        s[v["expert"]] = v["s"]
        b[v["expert"]] = v["bias"]
        names[v["expert"]] = name
    return fx, s, b, names


def test_illustrative_token_bias_selects_but_does_not_weight():
    fx, s, b, names = _illustrative()
    l = _logit(s)[None, :]
    r = oracle.route_from_logits(l, b)
    got = [names.get(int(e), "?") for e in r.idx[0]]
    assert sorted(got) == sorted(fx["expect_with_bias"])
    # E's selection score is 0.60 and its contribution uses 0.40.
    e_E = fx["candidates"]["E"]["expert"]
    assert r.c[0, e_E] == pytest.approx(fx["expect_E_selection_score"], abs=1e-12)
    assert r.s[0, e_E] == pytest.approx(fx["expect_E_contribution_score"], abs=1e-12)
    sel = np.array([fx["candidates"][n]["s"] for n in ["A", "B", "C", "E"]])
    expect_w = sel / (sel.sum() + 1e-6)
    np.testing.assert_allclose(r.w[0], expect_w, rtol=0, atol=1e-13)
    # Descending selection score: A (0.9), B (0.8), C (0.7), E (0.6).
    assert got == ["A", "B", "C", "E"]
    # Without the bias, D keeps its place.
    r0 = oracle.route_from_logits(l, np.zeros_like(b))
    assert sorted(names.get(int(e), "?") for e in r0.idx[0]) == sorted(fx["expect_without_bias"])
    # Using the selection score as the weight would give E 0.6 / 3.0 instead.
    assert r.w[0, 3] != pytest.approx(0.6 / (3.0 + 1e-6), abs=1e-3)


def test_weight_sum_slightly_below_one_closed_form():
    rng = np.random.default_rng(11)
    l = rng.normal(0, 0.9, size=(200, 64))
    b = rng.uniform(-0.25, 0.25, size=64)
    r = oracle.route_from_logits(l, b)
    S = np.take_along_axis(r.s, r.idx, 1).sum(1)
    total = r.w.sum(1)
    assert np.all(total < 1.0)
    np.testing.assert_allclose(1.0 - total, 1e-6 / (S + 1e-6), rtol=1e-6, atol=1e-15)
    # In bf16 the deficit (< 1e-6) rounds away: finite precision gives 1.0.
    assert np.all(oracle.round_bf16(total) == 1.0)


def test_sigmoid_and_silu_library_and_closed_forms():
    z = np.concatenate([np.linspace(-40, 40, 801), [0.0, 1e-300, -1e-300]])
    np.testing.assert_allclose(oracle.sigmoid(z), scipy.special.expit(z), rtol=1e-14, atol=0)
    assert oracle.sigmoid(np.array([0.0]))[0] == 0.5
    np.testing.assert_allclose(oracle.sigmoid(-z), 1 - oracle.sigmoid(z), atol=1e-15)
    t = torch.tensor(z, dtype=torch.float64)
    np.testing.assert_allclose(oracle.silu(z), torch.nn.functional.silu(t).numpy(), rtol=1e-14, atol=1e-300)


def test_router_logits_match_explicit_loops():
    rng = np.random.default_rng(3)
    X = rng.normal(size=(3, 7))
    W = rng.normal(size=(5, 7))
    l = oracle.router_logits(X, W)
    for t in range(3):
        for e in range(5):
            acc = 0.0
            for i in range(7):
                acc += X[t, i] * W[e, i]
            assert l[t, e] == pytest.approx(acc, abs=1e-12)


def test_selection_is_the_best_4_subset_brute_force():
    rng = np.random.default_rng(5)
    E, k = 64, 4
    subsets = np.array(list(combinations(range(E), k)))  # 635,376 subsets
    for trial in range(3):
        l = rng.normal(0, 0.9, size=(1, E))
        b = rng.uniform(-0.25, 0.25, size=E)
        r = oracle.route_from_logits(l, b)
        sums = r.c[0][subsets].sum(1)
        best = subsets[np.argmax(sums)]
        assert sorted(best.tolist()) == sorted(r.idx[0].tolist())
        # Descending order of selection scores inside the chosen set.
        assert np.all(np.diff(r.c[0, r.idx[0]]) <= 0)
        # Every chosen score beats every unchosen one.
        rest = np.setdiff1d(np.arange(E), r.idx[0])
        assert r.c[0, r.idx[0]].min() > r.c[0, rest].max()


def test_ties_go_to_lower_expert_id():
    E = 64
    s = np.full(E, 0.1)
    s[[10, 20, 30, 40, 50]] = 0.5
    r = oracle.route_from_logits(_logit(s)[None, :], np.zeros(E))
    assert r.idx[0].tolist() == [10, 20, 30, 40]
    assert r.margin[0] == 0.0


def test_bias_shift_invariance_and_unbiased_logit_order():
    rng = np.random.default_rng(7)
    l = rng.normal(0, 0.9, size=(50, 64))
    b = rng.uniform(-0.25, 0.25, size=64)
    r1 = oracle.route_from_logits(l, b)
    r2 = oracle.route_from_logits(l, b + 0.125)  # exact shift in binary
    np.testing.assert_array_equal(r1.idx, r2.idx)
    np.testing.assert_array_equal(r1.w, r2.w)
    # Without bias, sigmoid is monotone: the set is the top-4 raw logits.
    r0 = oracle.route_from_logits(l, np.zeros(64))
    np.testing.assert_array_equal(r0.idx, np.argsort(-l, axis=1, kind="stable")[:, :4])


def test_relabelling_experts_permutes_indices():
    rng = np.random.default_rng(9)
    X = rng.normal(size=(20, 32))
    W = rng.normal(0, 0.2, size=(64, 32))
    b = rng.uniform(-0.25, 0.25, size=64)
    perm = rng.permutation(64)
    r = oracle.route(X, W, b)
    rp = oracle.route(X, W[perm], b[perm])
    # Expert perm[i] of the original is expert i of the relabelled layer.
    np.testing.assert_array_equal(perm[rp.idx], r.idx)
    np.testing.assert_allclose(rp.w, r.w, rtol=0, atol=1e-15)


def test_bias_changes_most_selected_sets_at_workload_scale():
    """The guide: adding the bias after the activation can change the set."""
    rng = np.random.default_rng(13)
    l = rng.normal(0, 0.9, size=(512, 64))
    b = rng.uniform(-0.25, 0.25, size=64)
    r = oracle.route_from_logits(l, b)
    r0 = oracle.route_from_logits(l, np.zeros(64))
    differ = np.any(np.sort(r.idx, 1) != np.sort(r0.idx, 1), axis=1).mean()
    assert differ > 0.5


def test_valid_topk_sets_near_tie():
    E = 64
    c = np.linspace(0.0, 0.5, E)
    c[[1, 2, 3]] = [0.9, 0.8, 0.7]
    c[4] = 0.6
    c[5] = 0.6 + 5e-5     # within 1e-4 of expert 4
    sets = oracle.valid_topk_sets(c, 4, 1e-4)
    assert sorted(map(sorted, sets)) == [[1, 2, 3, 4], [1, 2, 3, 5]]
    assert oracle.valid_topk_sets(c, 4, 1e-6) == [[1, 2, 3, 5]]


def test_round_bf16_matches_library_conversion():
    rng = np.random.default_rng(17)
    v = np.concatenate([rng.normal(0, 3, 20000), rng.normal(0, 1e-3, 2000)]).astype(np.float32)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -7 * (1 + 2 ** -8)], dtype=np.float32)
    v = np.concatenate([v, ties])
    lib = torch.from_numpy(v).bfloat16().float().numpy().astype(np.float64)
    np.testing.assert_array_equal(oracle.round_bf16(v.astype(np.float64)), lib)
    assert oracle.round_bf16(np.array([1 + 2 ** -8]))[0] == 1.0            # tie to even
    assert oracle.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6  # tie to even (up)


def test_rmsnorm_closed_forms():
    x = np.array([[3.0, 4.0]])
    got = oracle.rmsnorm(x)
    np.testing.assert_allclose(got, x / math.sqrt(12.5 + 1e-6), rtol=1e-15)
    rng = np.random.default_rng(19)
    z = rng.normal(size=(8, 2048))
    y = oracle.rmsnorm(z)
    ms = np.mean(z * z, 1)
    np.testing.assert_allclose(np.mean(y * y, 1), ms / (ms + 1e-6), rtol=1e-12)
    # Scale invariance up to the epsilon term.
    np.testing.assert_allclose(oracle.rmsnorm(10 * z), y, rtol=1e-6)


def test_weights_for_set_closed_forms():
    """oracle.weights_for_set against the page's facts and the closed form:
    on the illustrative token E enters the weights with its unbiased 0.40
    (section "The router has two different scores"), the weights are the
    selected unbiased scores over their sum plus 1e-6, so they sum to
    S / (S + 1e-6) < 1, and they equal the router's own weights for the set
    it selects, in any order of the set."""
    fx, s, b, names = _illustrative()
    ids = {n: v["expert"] for n, v in fx["candidates"].items()}
    # Literal values: A 0.90, B 0.80, C 0.70, E 0.40 (E's score from the page).
    got = oracle.weights_for_set(s, [ids["A"], ids["B"], ids["C"], ids["E"]])
    den = 0.90 + 0.80 + 0.70 + 0.40 + 1e-6
    np.testing.assert_allclose(got, [0.90 / den, 0.80 / den, 0.70 / den, 0.40 / den], rtol=0, atol=1e-15)
    assert got[3] == pytest.approx(0.40 / 2.800001, abs=1e-15)   # not 0.60 / ...
    # Without the bias the set has D (0.55) in E's place.
    got_d = oracle.weights_for_set(s, [ids["A"], ids["B"], ids["C"], ids["D"]])
    np.testing.assert_allclose(got_d, np.array([0.90, 0.80, 0.70, 0.55]) / (2.95 + 1e-6), rtol=0,
                               atol=1e-15)
    # The set's order permutes the weights and nothing else.
    perm = oracle.weights_for_set(s, [ids["E"], ids["C"], ids["A"], ids["B"]])
    np.testing.assert_allclose(perm, got[[3, 2, 0, 1]], rtol=0, atol=1e-16)
    # Closed form of the sum on random tokens, and agreement with the router.
    rng = np.random.default_rng(5)
    l = rng.normal(0, 0.9, size=(64, 64))
    bias = rng.uniform(-0.25, 0.25, size=64)
    r = oracle.route_from_logits(l, bias)
    for t in range(64):
        S = [int(e) for e in r.idx[t]]
        w = oracle.weights_for_set(r.s[t], S)
        tot = float(np.sum(r.s[t, S]))
        assert w.sum() < 1.0
        assert 1.0 - w.sum() == pytest.approx(1e-6 / (tot + 1e-6), rel=1e-6)
        np.testing.assert_allclose(w, r.w[t], rtol=0, atol=1e-16)
        # A wrong set gives different weights (the function uses the set it is given).
        other = S[:3] + [next(e for e in range(64) if e not in S)]
        assert not np.allclose(oracle.weights_for_set(r.s[t], other), w, atol=1e-9)
