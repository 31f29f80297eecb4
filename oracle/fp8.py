"""CPU oracle of the FP8 block-scaled expert layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP
library and its Python binding never import, call or link it, and it shares
no code with them.

What it is: the MoE layer of ``oracle.moe`` with the expert weights and the
expert inputs quantised as the inferencekey.com page on the 24B reasoning
MoE describes the model's FP8 checkpoint (German edition, "Für Engineers"
part, the quantisation entry): compressed-tensors FP8_BLOCK -- weights in
FP8 statically, in blocks of 128 x 128; activations in FP8 dynamically, per
group of 128; the MoE router gates are not quantised.  The checkpoint's
listing names the weight dtype F8_E4M3.

Readings taken where the page is silent (each is a choice, not a fact of
the page):

* E4M3 is the OCP "E4M3FN" format: 1 sign, 4 exponent (bias 7) and 3
  mantissa bits; subnormals (exponent field 0) are m/8 * 2^-6; the largest
  finite magnitude is 448 (S.1111.110); S.1111.111 is NaN; no infinities.
* Encoding rounds to the nearest E4M3 value, ties to the even mantissa,
  saturating at +-448; a value that rounds to zero keeps its sign.
* A block or group with largest magnitude amax > 0 is stored as
  code = E4M3(fp32(x * fp32(448 / amax))) with dequantisation scale
  fp32(amax / 448) (fp32 IEEE arithmetic, round to nearest even, in exactly
  this order); amax = 0 gives code +-0 and scale 0.  The code is a rounded
  integer decision, so both the GPU path and this oracle take it in fp32
  with the same two operations.
* Weight blocks are 128 rows x 128 input columns of each of W_gate, W_up
  ([1536, 2048]: 12 x 16 blocks) and W_down ([2048, 1536]: 16 x 12 blocks).
* Activation groups are 128 consecutive input features of one row: a token
  row of X (16 groups) for gate/up, an expert hidden row for down (12
  groups).
* The hidden rows are rounded to bf16 (as in the bf16 layer) before they
  are quantised for the down projection.
* The router, its bias and the mixture weights are the bf16 layer's.

Everything after the quantisation runs in float64 on the dequantised values
(code value * scale), through ``oracle.moe``'s expert and combine
definitions.

Pins (tests/test_oracle_fp8.py): the E4M3 table against its closed-form
values; encoding against a brute-force nearest-value search, including
ties, subnormals and saturation; the quantisers' invariants (the block
maximum maps to +-448 exactly, error bounds, zero blocks); inputs already on
the E4M3 grid with amax = 448 quantise exactly, so the FP8 layer's hidden
rows equal the bf16 layer's; sparse = dense masked evaluation.
"""

from __future__ import annotations

import numpy as np

from .moe import LayerResult, group_by_expert, round_bf16, silu

E4M3_MAX = 448.0
WEIGHT_BLOCK = 128     # rows and columns of a weight block
ACT_GROUP = 128        # input features per activation group


def _e4m3_table() -> np.ndarray:
    """Value of every code 0..255 (NaN for the two NaN codes)."""
    v = np.empty(256)
    for q in range(256):
        s, e, m = q >> 7, (q >> 3) & 15, q & 7
        if e == 15 and m == 7:
            v[q] = np.nan
            continue
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        v[q] = -mag if s else mag
    return v


E4M3_VALUES = _e4m3_table()


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of E4M3 codes."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each (float32) value: ties to the even mantissa,
    saturating at +-448, zero keeps its sign; NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.where(np.isnan(x), 0.0, np.abs(x))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # Spacing of E4M3 values in the binade of |x| (subnormals share 2^-9).
    quantum = 2.0 ** (np.maximum(e, -6.0) - 3.0)
    mag = np.rint(a / quantum) * quantum          # np.rint: round half to even
    mag = np.minimum(mag, E4M3_MAX)
    # Code of a magnitude: exponent field and mantissa from its binade.
    me = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    normal = mag >= 2.0 ** -6
    exp_field = np.where(normal, me + 7, 0)
    mant = np.where(normal, mag / 2.0 ** me - 1.0, mag / 2.0 ** -6) * 8.0
    code = (exp_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(mag == 0, 0, code)
    code = code | (np.signbit(x).astype(np.int64) << 7)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def quantize_amax(x: np.ndarray, amax: np.ndarray):
    """Codes and scales of values x sharing the broadcast maximum amax (fp32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.asarray(amax, dtype=np.float32)
    nz = amax > 0
    with np.errstate(divide="ignore"):
        inv = np.where(nz, np.float32(E4M3_MAX) / np.where(nz, amax, np.float32(1)), np.float32(0))
    inv = inv.astype(np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    codes = e4m3_encode((x * inv).astype(np.float32))
    # amax = 0: x * 0 is +-0 already, so the codes keep the sign of zero.
    return codes, scale


def quantize_blocks(W, br: int = WEIGHT_BLOCK, bc: int = WEIGHT_BLOCK):
    """Static block quantisation of a weight matrix [R, C] (values exact in
    fp32): codes [R, C] uint8 and scales [R/br, C/bc] float32."""
    W = np.asarray(W, dtype=np.float32)
    R, C = W.shape
    blocks = W.reshape(R // br, br, C // bc, bc)
    amax = np.abs(blocks).max(axis=(1, 3))
    codes, _ = quantize_amax(blocks, amax[:, None, :, None])
    scales = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return codes.reshape(R, C), scales


def dequantize_blocks(codes, scales, br: int = WEIGHT_BLOCK, bc: int = WEIGHT_BLOCK) -> np.ndarray:
    R, C = codes.shape
    v = e4m3_decode(codes).reshape(R // br, br, C // bc, bc)
    return (v * scales.astype(np.float64)[:, None, :, None]).reshape(R, C)


def quantize_groups(X, g: int = ACT_GROUP):
    """Dynamic per-row group quantisation of activations [M, K] (values exact
    in fp32): codes [M, K] uint8 and scales [M, K/g] float32."""
    X = np.asarray(X, dtype=np.float32)
    M, K = X.shape
    groups = X.reshape(M, K // g, g)
    amax = np.abs(groups).max(axis=2)
    codes, _ = quantize_amax(groups, amax[:, :, None])
    scales = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return codes.reshape(M, K), scales


def dequantize_groups(codes, scales, g: int = ACT_GROUP) -> np.ndarray:
    M, K = codes.shape
    v = e4m3_decode(codes).reshape(M, K // g, g)
    return (v * scales.astype(np.float64)[:, :, None]).reshape(M, K)


def quantize_experts(W_gate, W_up, W_down) -> dict:
    """Block quantisation of all experts' weights, one matrix at a time."""
    E = W_gate.shape[0]
    out = {}
    for name, W in (("gate", W_gate), ("up", W_up), ("down", W_down)):
        qs = [quantize_blocks(W[e]) for e in range(E)]
        out[name + "_codes"] = np.stack([q[0] for q in qs])
        out[name + "_scales"] = np.stack([q[1] for q in qs])
    return out


def expert_hidden_fp8(Xq, q: dict, e: int, rounded: bool = True) -> np.ndarray:
    """Hidden rows of expert e for dequantised input rows Xq:
    silu(Xq W_gate^T) * (Xq W_up^T) with the dequantised weights, rounded to
    bf16 (the rounding point of the bf16 layer) unless ``rounded`` is False."""
    Wg = dequantize_blocks(q["gate_codes"][e], q["gate_scales"][e])
    Wu = dequantize_blocks(q["up_codes"][e], q["up_scales"][e])
    H = silu(Xq @ Wg.T) * (Xq @ Wu.T)
    return round_bf16(H) if rounded else H


def expert_down_fp8(H, q: dict, e: int) -> np.ndarray:
    """Output rows of expert e for bf16 hidden rows H: H quantised per group
    of 128, dequantised, times the dequantised W_down^T."""
    hc, hs = quantize_groups(H)
    Wd = dequantize_blocks(q["down_codes"][e], q["down_scales"][e])
    return dequantize_groups(hc, hs) @ Wd.T


def moe_apply_fp8(X, idx, w, q: dict) -> LayerResult:
    """The layer with FP8 experts, for given routing decisions.

    X: [N, 2048] exact bf16 values; q: the codes and scales of
    ``quantize_experts``.  Per expert: its rows of X quantised per group,
    G and U from the dequantised weights, H = silu(G) * U rounded to bf16,
    H quantised per group, Y from the dequantised W_down; then the weighted
    combine of ``oracle.moe``.
    """
    X = np.asarray(X, dtype=np.float64)
    idx = np.asarray(idx)
    w = np.asarray(w, dtype=np.float64)
    N, k = idx.shape
    E, ff, d = q["gate_codes"].shape
    g = group_by_expert(idx, E)
    # Token rows are quantised once; every selected expert sees the same codes.
    xc, xs = quantize_groups(X)
    Xq = dequantize_groups(xc, xs)
    H = np.zeros((N * k, ff))
    Y = np.zeros((N * k, d))
    for e in range(E):
        a, b = int(g.offsets[e]), int(g.offsets[e + 1])
        if a == b:
            continue
        H[a:b] = expert_hidden_fp8(Xq[g.row2tok[a:b]], q, e)
        Y[a:b] = expert_down_fp8(H[a:b], q, e)
    out = np.zeros((N, d))
    for j in range(k):
        out += w[:, j:j + 1] * Y[g.slot2row.reshape(N, k)[:, j]]
    return LayerResult(out=out, routing=None, grouping=g, H=H, Y=Y)


def dense_masked_forward_fp8(X, idx, w, q: dict) -> np.ndarray:
    """Every expert on every token (same quantisation), masked by the routing."""
    X = np.asarray(X, dtype=np.float64)
    N, k = np.asarray(idx).shape
    E = q["gate_codes"].shape[0]
    xc, xs = quantize_groups(X)
    Xq = dequantize_groups(xc, xs)
    out = np.zeros((N, X.shape[1]))
    for e in range(E):
        Ye = expert_down_fp8(expert_hidden_fp8(Xq, q, e), q, e)
        m = (np.asarray(idx) == e).astype(np.float64)
        out += ((m * w).sum(axis=1))[:, None] * Ye
    return out
