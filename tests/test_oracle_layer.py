"""Pins of the oracle's expert, grouping, combine and block steps.

The checks: pure-Python loops on tiny shapes, dense masked evaluation of
every expert, a one-expert special case built from torch's own SiLU,
linearity, token-permutation equivariance, negative controls that must fail
the parity gate, and the residual identity of a block.  CPU only.
"""

import numpy as np
import pytest
import torch

import oracle
from conftest import cached_layer

GATE = 2e-2  # max|err| <= GATE * RMS(out) is the parity bar on outputs


def _tiny(seed, N=5, E=6, d=7, ff=5, bias_scale=0.25):
    rng = np.random.default_rng(seed)
    X = rng.normal(size=(N, d))
    W_r = rng.normal(0, 0.5, size=(E, d))
    b = rng.uniform(-bias_scale, bias_scale, size=E)
    Wg = rng.normal(0, 0.5, size=(E, ff, d))
    Wu = rng.normal(0, 0.5, size=(E, ff, d))
    Wd = rng.normal(0, 0.5, size=(E, d, ff))
    return X, W_r, b, Wg, Wu, Wd


def _loops_layer(X, W_r, b, Wg, Wu, Wd, k, eps=1e-6):
    """The layer written out with scalar loops (independent of NumPy matmul)."""
    N, d = X.shape
    E, ff, _ = Wg.shape
    out = [[0.0] * d for _ in range(N)]
    for t in range(N):
        s, c = [], []
        for e in range(E):
            acc = 0.0
            for i in range(d):
                acc += X[t][i] * W_r[e][i]
            se = 1.0 / (1.0 + np.exp(-acc))
            s.append(se)
            c.append(se + b[e])
        chosen = sorted(range(E), key=lambda e: (-c[e], e))[:k]
        denom = sum(s[e] for e in chosen) + eps
        for e in chosen:
            wgt = s[e] / denom
            h = []
            for f in range(ff):
                g = sum(X[t][i] * Wg[e][f][i] for i in range(d))
                u = sum(X[t][i] * Wu[e][f][i] for i in range(d))
                h.append(g / (1.0 + np.exp(-g)) * u)
            for o in range(d):
                y = sum(h[f] * Wd[e][o][f] for f in range(ff))
                out[t][o] += wgt * y
    return np.array(out)


@pytest.mark.parametrize("seed,k", [(0, 2), (1, 3), (2, 4)])
def test_layer_matches_explicit_loops_on_tiny_shapes(seed, k):
    X, W_r, b, Wg, Wu, Wd = _tiny(seed)
    got = oracle.moe_forward(X, W_r, b, Wg, Wu, Wd, k=k).out
    ref = _loops_layer(X, W_r, b, Wg, Wu, Wd, k)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [3, 4])
def test_sparse_equals_dense_masked_tiny(seed):
    X, W_r, b, Wg, Wu, Wd = _tiny(seed, N=9, E=8, d=12, ff=10)
    sparse = oracle.moe_forward(X, W_r, b, Wg, Wu, Wd, k=4).out
    dense = oracle.dense_masked_forward(X, W_r, b, Wg, Wu, Wd, k=4)
    np.testing.assert_allclose(sparse, dense, rtol=1e-13, atol=1e-13)


def _layer_np(N, seed, skew=False, rows=None):
    p = cached_layer(N, seed, skew)
    X = oracle.block_input(p["z"].numpy())
    if rows is not None:
        X = X[rows]
    return (X, p["W_r"].float().numpy(), p["bias"].numpy(), p["W_gate"].float().numpy(),
            p["W_up"].float().numpy(), p["W_down"].float().numpy())


def test_sparse_equals_dense_masked_at_real_shapes():
    X, W_r, b, Wg, Wu, Wd = _layer_np(32, 0, rows=slice(0, 6))
    sparse = oracle.moe_forward(X, W_r, b, Wg, Wu, Wd).out
    dense = oracle.dense_masked_forward(X, W_r, b, Wg, Wu, Wd)
    scale = np.sqrt(np.mean(dense ** 2))
    assert np.max(np.abs(sparse - dense)) <= 1e-12 * scale


def test_single_expert_special_case_against_torch_silu():
    """E = 1, k = 1: out = s / (s + eps) * W_down (silu(W_gate x) * (W_up x))."""
    rng = np.random.default_rng(21)
    N, d, ff = 6, 16, 12
    X = rng.normal(size=(N, d))
    W_r = rng.normal(0, 0.3, size=(1, d))
    b = np.array([0.1])
    Wg = rng.normal(0, 0.3, size=(1, ff, d))
    Wu = rng.normal(0, 0.3, size=(1, ff, d))
    Wd = rng.normal(0, 0.3, size=(1, d, ff))
    got = oracle.moe_forward(X, W_r, b, Wg, Wu, Wd, k=1).out
    t = lambda a: torch.tensor(a, dtype=torch.float64)
    s = torch.sigmoid(t(X) @ t(W_r).T)
    mlp = (torch.nn.functional.silu(t(X) @ t(Wg[0]).T) * (t(X) @ t(Wu[0]).T)) @ t(Wd[0]).T
    ref = (s / (s + 1e-6)) * mlp
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-13, atol=1e-14)


def test_linear_in_down_projection_and_zero_down_gives_zero():
    X, W_r, b, Wg, Wu, Wd = _tiny(5, N=8, E=8, d=10, ff=6)
    base = oracle.moe_forward(X, W_r, b, Wg, Wu, Wd).out
    scaled = oracle.moe_forward(X, W_r, b, Wg, Wu, 2.5 * Wd).out
    np.testing.assert_allclose(scaled, 2.5 * base, rtol=1e-13, atol=1e-14)
    zero = oracle.moe_forward(X, W_r, b, Wg, Wu, 0 * Wd).out
    assert np.all(zero == 0.0)


def test_token_permutation_equivariance():
    X, W_r, b, Wg, Wu, Wd = _tiny(6, N=11, E=8, d=10, ff=6)
    perm = np.random.default_rng(0).permutation(11)
    a = oracle.moe_forward(X, W_r, b, Wg, Wu, Wd).out
    p = oracle.moe_forward(X[perm], W_r, b, Wg, Wu, Wd).out
    np.testing.assert_allclose(p, a[perm], rtol=1e-14, atol=1e-14)


def test_grouping_is_a_stable_counting_sort():
    rng = np.random.default_rng(23)
    N, E, k = 300, 64, 4
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(N)])
    g = oracle.group_by_expert(idx, E)
    assert g.counts.sum() == N * k
    np.testing.assert_array_equal(g.counts, [np.sum(idx == e) for e in range(E)])
    np.testing.assert_array_equal(g.offsets[1:], np.cumsum(g.counts))
    flat = idx.reshape(-1)
    # Bijection between rows and slots.
    assert sorted(g.row2slot.tolist()) == list(range(N * k))
    np.testing.assert_array_equal(g.slot2row[g.row2slot], np.arange(N * k))
    for e in range(E):
        rows = g.row2slot[g.offsets[e]:g.offsets[e + 1]]
        assert np.all(flat[rows] == e)
        assert np.all(np.diff(g.row2tok[g.offsets[e]:g.offsets[e + 1]]) > 0)


def _variant_out(X, W_r, b, Wg, Wu, Wd, which):
    l = oracle.router_logits(X, W_r)
    s = oracle.sigmoid(l)
    if which == "softmax":
        p = np.exp(l - l.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        r = oracle.route_from_logits(np.log(p) - np.log1p(-p), b)  # selection on softmax + bias
        sel = np.take_along_axis(p, r.idx, 1)
        return oracle.moe_apply(X, r.idx, sel / (sel.sum(1, keepdims=True) + 1e-6), Wg, Wu, Wd).out
    if which == "selection_as_weight":
        r = oracle.route_from_logits(l, b)
        sel = np.take_along_axis(r.c, r.idx, 1)
        return oracle.moe_apply(X, r.idx, sel / (sel.sum(1, keepdims=True) + 1e-6), Wg, Wu, Wd).out
    if which == "bias_before_sigmoid":
        r = oracle.route_from_logits(l + b[None, :], np.zeros_like(b))
        sel = np.take_along_axis(s, r.idx, 1)
        return oracle.moe_apply(X, r.idx, sel / (sel.sum(1, keepdims=True) + 1e-6), Wg, Wu, Wd).out
    if which == "no_bias":
        r = oracle.route_from_logits(l, np.zeros_like(b))
        return oracle.moe_apply(X, r.idx, r.w, Wg, Wu, Wd).out
    raise ValueError(which)


@pytest.mark.parametrize("which", ["softmax", "selection_as_weight", "bias_before_sigmoid", "no_bias"])
def test_negative_controls_fail_the_parity_gate(which):
    """The guide: each of these is a different model, so each must fail parity."""
    X, W_r, b, Wg, Wu, Wd = _layer_np(32, 0)
    ref = oracle.moe_forward(X, W_r, b, Wg, Wu, Wd).out
    bad = _variant_out(X, W_r, b, Wg, Wu, Wd, which)
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(bad - ref)) > GATE * rms * 5


def test_bf16_output_rounding_stays_inside_the_gate():
    """Rounding points of the HIP path (H to bf16) must leave room in the gate."""
    X, W_r, b, Wg, Wu, Wd = _layer_np(32, 0)
    ref = oracle.moe_forward(X, W_r, b, Wg, Wu, Wd)
    g = ref.grouping
    Hq = oracle.round_bf16(ref.H)
    Y = np.zeros_like(ref.Y)
    for e in range(64):
        a, c = int(g.offsets[e]), int(g.offsets[e + 1])
        if a < c:
            Y[a:c] = Hq[a:c] @ Wd[e].astype(np.float64).T
    out = np.zeros_like(ref.out)
    for j in range(4):
        out += ref.routing.w[:, j:j + 1] * Y[g.slot2row.reshape(-1, 4)[:, j]]
    rms = np.sqrt(np.mean(ref.out ** 2))
    assert np.max(np.abs(out - ref.out)) < 0.5 * GATE * rms


def test_block_residual_identity_and_composition():
    rng = np.random.default_rng(29)
    N, E, d, ff = 7, 8, 16, 6
    x = rng.normal(size=(N, d))
    W_r = rng.normal(0, 0.3, size=(E, d))
    b = rng.uniform(-0.25, 0.25, size=E)
    Wg = rng.normal(0, 0.3, size=(E, ff, d))
    Wu = rng.normal(0, 0.3, size=(E, ff, d))
    Wd = rng.normal(0, 0.3, size=(E, d, ff))
    assert np.all(oracle.block_forward(x, W_r, b, Wg, Wu, 0 * Wd) == x)
    X = oracle.round_bf16(oracle.rmsnorm(x))
    np.testing.assert_allclose(oracle.block_forward(x, W_r, b, Wg, Wu, Wd),
                               x + oracle.moe_forward(X, W_r, b, Wg, Wu, Wd).out, rtol=0, atol=0)


def test_expert_weight_count_and_flop_constants():
    """Guide: 3 x 2048 x 1536 = 9,437,184 weights per expert; selected-expert
    products cost 2 x 38 x 4 x 3 x 2048 x 1536 ~ 2.869 GFLOP per token."""
    per_expert = 3 * oracle.HIDDEN * oracle.FF
    assert per_expert == 9_437_184
    assert 2 * 38 * oracle.TOP_K * per_expert == pytest.approx(2.869e9, rel=1e-3)
