"""Parity checks between the HIP path and the oracle (test helpers).

Bar: selected experts bit-exact wherever the oracle's 4th/5th selection-score
margin exceeds 1e-4; elsewhere the HIP set must be one of the sets the oracle
accepts within 1e-4, and is then checked against the oracle's output for
that set.  Outputs within max|err| <= 2e-2 * RMS(oracle output).
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

MARGIN = 1e-4
OUT_GATE = 2e-2
W_ATOL = 2e-6  # fp32 sigmoid + normalisation vs float64
# The FP8 layer's grouped kernels multiply on the gfx950 FP8 matrix core
# (32x32x64 E4M3), whose sums are not fp32 sums of the exact products: it
# aligns the products of a step before adding them and drops the bits below
# the alignment.  Measured (probes of single and of 32 chained steps, random
# and normally distributed codes): a step's result lies within 2^-11.7 of
# the sum of its 64 products' magnitudes of the exact accumulator-plus-sum,
# after half an fp32 ulp of the result.  The stage checks of that path allow
# FP8_CORE_ACC times the sum of the magnitudes of a value's products.
FP8_CORE_ACC = 2.0 ** -11


def fp8_core_hidden_bound(Xq: np.ndarray, q: dict, e: int) -> np.ndarray:
    """Bound of |H - H64| that the FP8 matrix core's summation adds, for the
    dequantised token rows Xq of expert e: first order in the errors of G and
    U (each FP8_CORE_ACC times its sum of product magnitudes), plus the
    second-order terms (|silu''| <= 1/2, |silu'| <= 1.1)."""
    from oracle import fp8
    Wg = fp8.dequantize_blocks(q["gate_codes"][e], q["gate_scales"][e])
    Wu = fp8.dequantize_blocks(q["up_codes"][e], q["up_scales"][e])
    G, U = Xq @ Wg.T, Xq @ Wu.T
    dG = FP8_CORE_ACC * (np.abs(Xq) @ np.abs(Wg).T)
    dU = FP8_CORE_ACC * (np.abs(Xq) @ np.abs(Wu).T)
    sig = 1.0 / (1.0 + np.exp(-G))
    silu = G * sig
    dsilu = sig * (1.0 + G * (1.0 - sig))
    return (np.abs(dsilu * U) * dG + np.abs(silu) * dU
            + 1.1 * dG * dU + 0.25 * dG ** 2 * (np.abs(U) + dU))


def fp8_core_down_bound(H: np.ndarray, q: dict, e: int) -> np.ndarray:
    """Bound of |Y - Y_ref| that the FP8 matrix core's summation adds to the
    down step of expert e on bf16 hidden rows H."""
    from oracle import fp8
    Hq = fp8.dequantize_groups(*fp8.quantize_groups(H))
    Wd = fp8.dequantize_blocks(q["down_codes"][e], q["down_scales"][e])
    return FP8_CORE_ACC * (np.abs(Hq) @ np.abs(Wd).T)


def oracle_inputs(layer: dict) -> dict:
    """Oracle-side arrays of a workload (exact values of the bf16 inputs)."""
    return dict(
        X=oracle.block_input(layer["z"].numpy()),
        W_r=layer["W_r"].float().numpy(),
        bias=layer["bias"].numpy(),
        W_gate=layer["W_gate"].float().numpy(),
        W_up=layer["W_up"].float().numpy(),
        W_down=layer["W_down"].float().numpy(),
    )


def device_weights(layer: dict, device="cuda") -> dict:
    """Router, bias and packed expert weights on the device (packed by the library)."""
    import biased_sigmoid_top_amd as moe
    Wg, Wu = layer["W_gate"].to(device), layer["W_up"].to(device)
    W_gateup = moe.pack_gateup(Wg, Wu)
    del Wg, Wu
    Wd = layer["W_down"].contiguous().to(device)
    W_down = moe.pack_down(Wd)
    del Wd
    return dict(W_r=layer["W_r"].to(device), bias=layer["bias"].to(device),
                W_gateup=W_gateup, W_down=W_down)


def device_inputs(layer: dict, X: np.ndarray, device="cuda") -> dict:
    """Device tensors for the HIP path; X is the oracle's bf16-valued input."""
    d = device_weights(layer, device)
    d["X"] = torch.from_numpy(X).to(torch.bfloat16).to(device)
    return d


def check_route(idx_gpu: np.ndarray, w_gpu: np.ndarray, r: oracle.Routing, tokens=None):
    """Returns {token: accepted set} for tokens whose set differs (near ties).

    Raises AssertionError on any violation of the bar.
    """
    N = idx_gpu.shape[0]
    tokens = range(N) if tokens is None else tokens
    alt = {}
    for t in tokens:
        g = [int(e) for e in idx_gpu[t]]
        o = [int(e) for e in r.idx[t]]
        assert len(set(g)) == 4 and all(0 <= e < 64 for e in g), (t, g)
        if sorted(g) != sorted(o):
            assert r.margin[t] <= MARGIN, f"token {t}: set {g} != oracle {o}, margin {r.margin[t]:.3e}"
            sets = oracle.valid_topk_sets(r.c[t], 4, MARGIN)
            match = [S for S in sets if sorted(S) == sorted(g)]
            assert match, f"token {t}: {g} is not an accepted near-tie set {sets}"
            alt[t] = match[0]
        S = alt.get(t, o)
        expect = dict(zip(S, oracle.weights_for_set(r.s[t], S)))
        got = dict(zip(g, w_gpu[t].astype(np.float64)))
        for e in S:
            assert abs(got[e] - expect[e]) <= W_ATOL, (t, e, got[e], expect[e])
        # Descending selection score (within the margin) in the HIP order.
        cs = r.c[t, g]
        assert np.all(np.diff(cs) <= MARGIN), (t, g, cs)
    return alt


def expected_outputs(inp: dict, r: oracle.Routing, tokens: np.ndarray, alt: dict) -> np.ndarray:
    """Oracle output rows for `tokens`, using the accepted set where it differs."""
    idx = r.idx[tokens].copy()
    w = r.w[tokens].copy()
    for i, t in enumerate(tokens):
        if int(t) in alt:
            S = alt[int(t)]
            idx[i] = S
            w[i] = oracle.weights_for_set(r.s[t], S)
    return oracle.moe_apply(inp["X"][tokens], idx, w, inp["W_gate"], inp["W_up"],
                            inp["W_down"]).out


def check_out(out_gpu: np.ndarray, expect: np.ndarray, rms: float | None = None) -> float:
    """Asserts max|err| <= 2e-2 * RMS(oracle); returns the error ratio."""
    if rms is None:
        rms = float(np.sqrt(np.mean(expect ** 2)))
    err = float(np.max(np.abs(out_gpu.astype(np.float64) - expect)))
    assert np.all(np.isfinite(out_gpu)), "non-finite outputs"
    assert err <= OUT_GATE * rms, f"max|err| {err:.4e} > {OUT_GATE} * RMS {rms:.4e}"
    return err / rms


def check_grouping_valid(idx: np.ndarray, offsets: np.ndarray, row2slot: np.ndarray) -> None:
    """The grouping is THE stable counting sort of idx (it is unique)."""
    N = idx.shape[0]
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=64)
    assert offsets[0] == 0 and offsets[64] == 4 * N
    np.testing.assert_array_equal(np.diff(offsets), counts)
    r2s = row2slot.astype(np.int64)
    assert np.array_equal(np.sort(r2s), np.arange(4 * N)), "row2slot is not a permutation"
    for e in range(64):
        a, b = offsets[e], offsets[e + 1]
        assert np.all(flat[r2s[a:b]] == e)
        assert np.all(np.diff(r2s[a:b] // 4) > 0), f"expert {e} rows not in token order"


def sanitize_routing(idx: np.ndarray) -> np.ndarray:
    """Host mirror of the rule the expert-path entry points apply to given
    selections: ids modulo 64; an id that repeats an earlier (final) id of
    its token becomes the lowest id that is neither among the token's other
    ids -- earlier ones as replaced, later ones as given."""
    v = (np.asarray(idx, dtype=np.int64) & 63).astype(np.int32)
    for row in v:
        for q in range(1, 4):
            if row[q] in row[:q]:
                others = {int(row[p]) for p in range(4) if p != q}
                row[q] = min(e for e in range(64) if e not in others)
    return v


def oracle_fp8_experts(inp: dict, workers: int = 8) -> dict:
    """oracle.fp8.quantize_experts of a workload's expert weights, one
    (matrix, expert) block quantisation per task on a thread pool (numpy
    releases the GIL in the element-wise work)."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import fp8
    jobs = [(name, e) for name in ("gate", "up", "down") for e in range(inp["W_gate"].shape[0])]
    src = {"gate": inp["W_gate"], "up": inp["W_up"], "down": inp["W_down"]}
    with ThreadPoolExecutor(workers) as pool:
        res = list(pool.map(lambda j: fp8.quantize_blocks(src[j[0]][j[1]]), jobs))
    q = {}
    for name in ("gate", "up", "down"):
        qs = [r for (n, _), r in zip(jobs, res) if n == name]
        q[name + "_codes"] = np.stack([c for c, _ in qs])
        q[name + "_scales"] = np.stack([s for _, s in qs])
    return q


def fp8_output_check(out: np.ndarray, idx: np.ndarray, w: np.ndarray, H_gpu: np.ndarray,
                     X: np.ndarray, q: dict) -> dict:
    """Output parity of the FP8 layer for the GPU's selections idx and weights
    w (slot order t * 4 + j everywhere).

    The E4M3 codes of a hidden row are an integer decision taken from its
    bf16 values, which come from fp32 sums on the GPU and from float64 on the
    oracle; where the two round H to neighbouring bf16 values, a code can
    land on the neighbouring E4M3 value (and a group maximum moves its whole
    group's scale).  So the output is gated against the oracle's down step
    and combine applied to the GPU's own H (both sides decide the codes from
    the same values), within OUT_GATE * RMS; the fully independent oracle
    result is also compared, and must pass the same gate whenever no code
    differs.  Returns the ratios and the number of differing codes."""
    from oracle import fp8
    N = idx.shape[0]
    flat = idx.reshape(-1)
    xc, xs = fp8.quantize_groups(X)
    Xq = fp8.dequantize_groups(xc, xs)
    H_ref = np.zeros_like(H_gpu)
    Y_same = np.zeros((4 * N, X.shape[1]))
    for e in np.unique(flat):
        rows = np.nonzero(flat == e)[0]
        H_ref[rows] = fp8.expert_hidden_fp8(Xq[rows // 4], q, int(e))
        Y_same[rows] = fp8.expert_down_fp8(H_gpu[rows], q, int(e))
    out_same = (w[:, :, None] * Y_same.reshape(N, 4, -1)).sum(axis=1)
    ref = fp8.moe_apply_fp8(X, idx, w, q).out
    gc, gs = fp8.quantize_groups(H_gpu)
    rc, rs = fp8.quantize_groups(H_ref)
    code_flips = int(np.sum(gc != rc))
    scale_flips = int(np.sum(gs != rs))
    rms_same = float(np.sqrt(np.mean(out_same ** 2)))
    rms = float(np.sqrt(np.mean(ref ** 2)))
    res = dict(same_codes=float(np.max(np.abs(out - out_same))) / rms_same,
               end_to_end=float(np.max(np.abs(out - ref))) / rms,
               h_differs=int(np.sum(H_gpu != H_ref)), code_flips=code_flips, scale_flips=scale_flips)
    assert np.all(np.isfinite(out)), "non-finite outputs"
    assert res["same_codes"] <= OUT_GATE, res
    if code_flips == 0 and scale_flips == 0:
        assert res["end_to_end"] <= OUT_GATE, res
    return res
