"""Pins of the FP8 oracle (oracle/fp8.py) against what the format and the
quantisation definitions fix, independently of the oracle's own code."""

import numpy as np
import pytest

import oracle
from oracle import fp8


def test_e4m3_table_closed_form_values():
    v = fp8.E4M3_VALUES
    # Values fixed by the E4M3FN definition (bias 7, 3 mantissa bits).
    assert v[0x00] == 0.0 and np.signbit(v[0x80]) and v[0x80] == 0.0
    assert v[0x01] == 2.0 ** -9            # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert v[0x08] == 2.0 ** -6            # smallest normal
    assert v[0x38] == 1.0 and v[0x3C] == 1.5 and v[0x40] == 2.0 and v[0x30] == 0.5
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    finite = v[~np.isnan(v)]
    assert finite.size == 254
    pos = v[0x00:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes are ordered by value"
    np.testing.assert_array_equal(v[0x80:0xFF], -pos)


def _brute_nearest(x: float) -> int:
    """Nearest finite E4M3 value by exhaustive search; ties to the even
    mantissa; beyond 448 the largest finite value (saturation)."""
    v = fp8.E4M3_VALUES
    best, bd = None, np.inf
    for q in range(256):
        if np.isnan(v[q]) or (q & 0x80):
            continue
        d = abs(v[q] - abs(x))
        if d < bd or (d == bd and (q & 1) == 0):
            best, bd = q, d
    return best | (0x80 if np.signbit(x) else 0)


def test_encode_matches_exhaustive_nearest_value():
    rng = np.random.default_rng(0)
    xs = [0.0, -0.0, 1e-9, -1e-9, 448.0, 449.0, 464.0, 465.0, 1e6, -1e6,
          2.0 ** -10, 2.0 ** -9 * 0.5, 2.0 ** -9 * 1.5, 2.0 ** -6 * 0.999]
    # Every midpoint between neighbouring positive values (exact ties).
    pos = fp8.E4M3_VALUES[0x00:0x7F]
    xs += list((pos[:-1] + pos[1:]) / 2) + list(-(pos[:-1] + pos[1:]) / 2)
    xs += list(rng.standard_normal(400) * np.exp(rng.uniform(-12, 7, 400)))
    xs = np.array(xs, dtype=np.float32)
    got = fp8.e4m3_encode(xs)
    want = np.array([_brute_nearest(float(x)) for x in xs], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def test_encode_ties_go_to_the_even_mantissa():
    enc = fp8.e4m3_encode
    assert enc(np.float32(1.0625)) == 0x38      # between 1.0 (m=0) and 1.125 (m=1)
    assert enc(np.float32(1.1875)) == 0x3A      # between 1.125 (m=1) and 1.25 (m=2)
    assert enc(np.float32(1.9375)) == 0x40      # between 1.875 and 2.0: the next binade
    assert enc(np.float32(464.0)) == 0x7E       # between 448 and (absent) 480: saturates
    assert enc(np.float32(np.nan)) == 0x7F


def test_block_quantisation_invariants():
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    W[5, 7] = 0.5                                # a block maximum
    codes, scales = fp8.quantize_blocks(W)
    assert codes.shape == W.shape and scales.shape == (2, 3)
    assert codes[5, 7] == 0x7E                   # the maximum maps to +448 exactly
    assert scales[0, 0] == np.float32(0.5) / np.float32(448)
    Wq = fp8.dequantize_blocks(codes, scales)
    # E4M3 keeps 4 significant bits: relative error <= 2^-4 above the
    # subnormal range of each block, absolute <= half a subnormal step below.
    blk_scale = np.repeat(np.repeat(scales.astype(np.float64), 128, 0), 128, 1)
    bound = np.maximum(np.abs(W) * 2.0 ** -4, blk_scale * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(Wq - W) <= bound)
    Z = np.zeros((128, 128), dtype=np.float32)
    zc, zs = fp8.quantize_blocks(Z)
    assert np.all(zc == 0) and np.all(zs == 0)


def test_group_quantisation_of_grid_values_is_exact():
    """Values on the E4M3 grid whose group maximum is 448 are stored exactly."""
    rng = np.random.default_rng(2)
    pos = fp8.E4M3_VALUES[0x00:0x7F]
    X = rng.choice(pos, size=(3, 256)) * rng.choice([-1.0, 1.0], size=(3, 256))
    X[:, 0] = 448.0
    X[:, 128] = -448.0
    codes, scales = fp8.quantize_groups(X)
    assert np.all(scales == 1.0)
    np.testing.assert_array_equal(fp8.dequantize_groups(codes, scales), X)


def _tiny_fp8_layer(seed, E=6, d=256, ff=384, N=9, k=2):
    rng = np.random.default_rng(seed)
    X = oracle.round_bf16(rng.standard_normal((N, d)))
    Wg = oracle.round_bf16(rng.standard_normal((E, ff, d)) * 0.05)
    Wu = oracle.round_bf16(rng.standard_normal((E, ff, d)) * 0.05)
    Wd = oracle.round_bf16(rng.standard_normal((E, d, ff)) * 0.05)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(N)])
    w = rng.uniform(0.1, 0.5, size=(N, k))
    return X, Wg, Wu, Wd, idx, w


def test_fp8_layer_sparse_equals_dense_masked():
    X, Wg, Wu, Wd, idx, w = _tiny_fp8_layer(3)
    q = fp8.quantize_experts(Wg, Wu, Wd)
    sparse = fp8.moe_apply_fp8(X, idx, w, q).out
    dense = fp8.dense_masked_forward_fp8(X, idx, w, q)
    np.testing.assert_allclose(sparse, dense, rtol=1e-12, atol=1e-12)


def test_grid_weights_give_the_bf16_layer_hidden_rows():
    """Weights and inputs on the E4M3 grid with block and group maxima of 448
    quantise without error, so the FP8 layer's hidden rows (before their own
    quantisation) are the bf16 layer's."""
    rng = np.random.default_rng(4)
    pos = fp8.E4M3_VALUES[0x30:0x48]               # 0.5 .. 3.75: a few binades
    E, d, ff, N, k = 3, 256, 256, 5, 2
    sgn = lambda shape: rng.choice([-1.0, 1.0], size=shape)
    X = rng.choice(pos, size=(N, d)) * sgn((N, d)) / 64.0
    X[:, ::128] = 448.0 / 64.0                     # each group's maximum is 448 / 64
    Wg = rng.choice(pos, size=(E, ff, d)) * sgn((E, ff, d))
    Wu = rng.choice(pos, size=(E, ff, d)) * sgn((E, ff, d))
    Wd = rng.choice(pos, size=(E, d, ff)) * sgn((E, d, ff))
    for W in (Wg, Wu, Wd):
        W[:, ::128, ::128] = 448.0                 # every block holds a 448
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(N)])
    w = np.full((N, k), 0.5)
    q = fp8.quantize_experts(Wg, Wu, Wd)
    for name, W in (("gate", Wg), ("up", Wu), ("down", Wd)):
        for e in range(E):
            np.testing.assert_array_equal(
                fp8.dequantize_blocks(q[name + "_codes"][e], q[name + "_scales"][e]), W[e])
    # X's groups have maximum 7 (448 / 64): scale 1/64, still exact.
    xc, xs = fp8.quantize_groups(X)
    np.testing.assert_array_equal(fp8.dequantize_groups(xc, xs), X)
    got = fp8.moe_apply_fp8(X, idx, w, q)
    ref = oracle.moe_apply(X, idx, w, Wg, Wu, Wd)
    np.testing.assert_array_equal(got.H, oracle.round_bf16(ref.H))


@pytest.mark.parametrize("seed", [5, 6])
def test_fp8_layer_is_close_to_the_bf16_layer(seed):
    """Negative control and sanity: FP8 quantisation changes the output by a
    few percent of its RMS, not more, and not zero."""
    X, Wg, Wu, Wd, idx, w = _tiny_fp8_layer(seed)
    q = fp8.quantize_experts(Wg, Wu, Wd)
    a = fp8.moe_apply_fp8(X, idx, w, q).out
    b = oracle.moe_apply(X, idx, w, Wg, Wu, Wd).out
    rel = np.sqrt(np.mean((a - b) ** 2)) / np.sqrt(np.mean(b ** 2))
    assert 1e-3 < rel < 0.1


def _grid_values(rng, n):
    """n random E4M3 normal values built from the format's definition,
    +-(1 + m/8) * 2^e with e in [-6, 7] (all below 448, exact in fp32)."""
    m = rng.integers(0, 8, n)
    e = rng.integers(-6, 8, n)
    sgn = rng.choice([-1.0, 1.0], n)
    return sgn * (1.0 + m / 8.0) * np.exp2(e)


def test_down_step_quantises_hidden_rows_and_weights_exactly():
    """fp8.expert_down_fp8 on hand-checked values.  Every group or block
    maximum is 448 * 2^-k, so its scale 2^-k and 448 / amax are exact; each
    off-grid value is listed with the E4M3 value the format's spacing rounds
    it to (round to nearest; no value sits near a midpoint).  The products
    and sums of these dyadic values are exact in float64, so the down step
    must equal the hand-dequantised product bit for bit.  A down step that
    skipped the quantisation of H, used another group size, or dropped a
    scale would give a different result."""
    # (raw value, dequantised value) per group; group = 128 columns.
    H_cases = {
        (0, 0): [(448.0, 448.0), (1.03, 1.0), (2.3, 2.25), (-5.1, -5.0), (300.0, 288.0),
                 (0.0101, 5 * 2.0 ** -9)],                      # scale 1; 0.0101 is subnormal
        (0, 1): [(56.0, 56.0), (1.03, 1.0), (3.3, 3.25), (-0.7, -0.6875)],   # 56 = 448 / 8
        (1, 0): [(-7.0, -7.0), (0.1, 0.1015625), (1.0, 1.0)],              # 7 = 448 / 64
        (1, 1): [],                                                          # all zero: scale 0
        (2, 0): [(224.0, 224.0), (0.33, 0.34375)],                           # 224 = 448 / 2
        (2, 1): [(-28.0, -28.0), (2.2, 2.25)],                               # 28 = 448 / 16
    }
    H = np.zeros((3, 256))
    H_deq = np.zeros((3, 256))
    for (row, grp), vals in H_cases.items():
        for i, (raw, deq) in enumerate(vals):
            col = grp * 128 + 7 * i + 3
            H[row, col] = raw
            H_deq[row, col] = deq
    rng = np.random.default_rng(3)
    W = np.zeros((128, 256))
    W[:, :128] = _grid_values(rng, 128 * 128).reshape(128, 128)          # block scale 1
    W[:, 128:] = 0.25 * _grid_values(rng, 128 * 128).reshape(128, 128)  # block scale 1/4
    W[0, 0] = 448.0
    W[5, 200] = 112.0                                                    # 448 / 4
    W_deq = W.copy()
    W[1, 10], W_deq[1, 10] = 1.03, 1.0         # scale 1: 1.03 -> 1.0
    W[9, 131], W_deq[9, 131] = 0.3, 0.3125     # scale 1/4: 1.2 -> 1.25
    codes, scales = fp8.quantize_blocks(W)
    q = {"down_codes": codes[None], "down_scales": scales[None]}
    got = fp8.expert_down_fp8(H, q, 0)
    want = H_deq @ W_deq.T
    np.testing.assert_array_equal(got, want)
    # The quantisation matters: the unquantised product is another result.
    assert not np.array_equal(got, H @ W_deq.T)
    assert not np.array_equal(got, H_deq @ W.T)
