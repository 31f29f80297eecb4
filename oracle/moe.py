"""CPU oracle for the biased-sigmoid top-4 sparse feed-forward (MoE) layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP
library and its Python binding never import, call or link it, and it shares
no code with them.

What it is: a plain, slow, float64 NumPy statement of what the layer computes,
written from the English edition of the flozi.net guide "LFM2.5-24B-A2B:
Biased Routing, Short Convolutions and Ten KV Caches" (cited below as
"the guide"), section by section:

* "The exact checkpoint": a block applies RMS normalisation before its
  feed-forward network and adds a residual after it.
* "The router has two different scores": hidden states flattened to
  X[N, 2048]; a 64 x 2048 router gives 64 logits per token; sigmoid is
  applied to each logit on its own; a stored 64-element bias takes part in
  the top-4 selection only and is added after the activation; the mixture
  weights are the unbiased sigmoid scores, normalised with an epsilon so
  that they sum to slightly less than one, routed scale 1; every selected
  expert is a gated SiLU MLP with three matrices (2048 -> 1536 -> 2048).
* "What to verify in a deployment": the expert path groups tokens by
  expert and accumulates the weighted expert outputs.

Inputs are taken at their exact values (bf16 weights and activations widen
to float64 without error); every step runs in float64; nothing is blocked,
fused or reordered beyond what the definitions state.  NumPy's matmul,
exp and argsort are the only library primitives.

Readings taken where the guide is silent (each is a choice, not a fact of
the guide): epsilon = 1e-6 and it enters as sum + eps in the denominator;
the sum runs over the k selected scores; equal selection scores are broken
towards the lower expert id; silu(z) = z * sigmoid(z) is applied to the
gate projection; weights are stored [out_features, in_features]; RMSNorm is
x / sqrt(mean(x^2) + 1e-6) with unit weight.

Pins (tests/test_oracle_*.py): the guide's illustrative token, the closed
form of the weight sum, negative controls, brute force over all 4-subsets,
dense masked evaluation of every expert, explicit-loop evaluation on tiny
shapes, invariants and library special cases.  Parity unpinned: nothing the
guide fixes about trained weights (none exist here) -- only the synthetic
workloads are covered.
"""

from __future__ import annotations

from dataclasses import dataclass
from itertools import combinations

import numpy as np

HIDDEN = 2048          # model width, guide: "The exact checkpoint"
EXPERTS = 64           # router rows, guide: "The router has two different scores"
TOP_K = 4              # four of 64 experts per token
FF = 1536              # expert intermediate width (3 x 2048 x 1536 weights)
ROUTER_EPS = 1e-6      # epsilon of the weight normalisation (value not printed)
ROUTED_SCALE = 1.0     # routed scaling factor
RMS_EPS = 1e-6         # RMSNorm epsilon


def f64(a) -> np.ndarray:
    """Exact widening of any float array (bf16 values held in f32, f32, f64)."""
    return np.asarray(a, dtype=np.float64)


def sigmoid(z) -> np.ndarray:
    """Logistic function 1 / (1 + exp(-z)), evaluated without overflow."""
    z = f64(z)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def silu(z) -> np.ndarray:
    """SiLU z * sigmoid(z), the activation of the gated expert MLP."""
    z = f64(z)
    return z * sigmoid(z)


def rmsnorm(x, eps: float = RMS_EPS) -> np.ndarray:
    """RMS normalisation over the last axis with unit weight.

    Guide, "The exact checkpoint": RMS normalisation before the feed-forward
    network.  Form x / sqrt(mean(x^2) + eps).
    """
    x = f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bf16 keeps 8 significant bits.  With a = m * 2**e, 0.5 <= |m| < 1,
    m * 256 is exact in float64 and np.rint rounds it half-to-even.  Values
    stay in the normal range for every workload here.
    """
    m, e = np.frexp(f64(a))
    return np.ldexp(np.rint(m * 256.0), e - 8)


@dataclass
class Routing:
    idx: np.ndarray     # [N, k] int64, selected experts, descending selection score
    w: np.ndarray       # [N, k] float64 mixture weights
    s: np.ndarray       # [N, E] unbiased sigmoid scores
    c: np.ndarray       # [N, E] selection scores s + bias
    margin: np.ndarray  # [N] c of the k-th minus c of the (k+1)-th expert


def router_logits(X, W_r) -> np.ndarray:
    """l = X W_r^T: one logit per expert (router matrix [E, d])."""
    return f64(X) @ f64(W_r).T


def route_from_logits(l, bias, k: int = TOP_K, eps: float = ROUTER_EPS,
                      scale: float = ROUTED_SCALE) -> Routing:
    """Biased top-k selection and unbiased, normalised mixture weights.

    Guide, "The router has two different scores":
      s = sigmoid(l) per logit;
      c = s + bias (bias added after the activation, selection only);
      the k largest c are selected (ties: lower expert id first);
      w_j = s[idx_j] / (sum_j' s[idx_j'] + eps) * scale.
    """
    l = f64(l)
    s = sigmoid(l)
    c = s + f64(bias)[None, :]
    order = np.argsort(-c, axis=1, kind="stable")
    idx = order[:, :k]
    sel = np.take_along_axis(s, idx, axis=1)
    w = sel / (sel.sum(axis=1, keepdims=True) + eps) * scale
    ck = np.take_along_axis(c, order[:, k - 1:k], axis=1)[:, 0]
    if c.shape[1] > k:
        ck1 = np.take_along_axis(c, order[:, k:k + 1], axis=1)[:, 0]
        margin = ck - ck1
    else:
        margin = np.full(c.shape[0], np.inf)
    return Routing(idx=idx, w=w, s=s, c=c, margin=margin)


def route(X, W_r, bias, k: int = TOP_K) -> Routing:
    """Router of the layer: logits, sigmoid, biased selection, weights."""
    return route_from_logits(router_logits(X, W_r), bias, k=k)


def weights_for_set(s_row, S, eps: float = ROUTER_EPS, scale: float = ROUTED_SCALE):
    """Mixture weights of one token for a given selected set S (any order)."""
    sel = f64(s_row)[list(S)]
    return sel / (sel.sum() + eps) * scale


def valid_topk_sets(c_row, k: int = TOP_K, tol: float = 1e-4):
    """Every k-set S with min c[S] >= max c[not S] - tol, in descending-c order.

    Where two selection scores lie within tol of each other, the top-k set
    is decided by rounding; all such sets are correct answers.
    """
    c_row = f64(c_row)
    E = c_row.shape[0]
    order = np.argsort(-c_row, kind="stable")
    ck1 = c_row[order[k]] if E > k else -np.inf
    ck = c_row[order[k - 1]]
    sure = [int(e) for e in order if c_row[e] > ck1 + tol]
    band = [int(e) for e in order if c_row[e] >= ck - tol and int(e) not in sure]
    out = []
    for extra in combinations(band, k - len(sure)):
        S = sure + list(extra)
        rest = [e for e in range(E) if e not in S]
        if min(c_row[S]) >= max(c_row[rest]) - tol if rest else True:
            out.append(sorted(S, key=lambda e: (-c_row[e], e)))
    return out


@dataclass
class Grouping:
    counts: np.ndarray    # [E] slots routed to each expert
    offsets: np.ndarray   # [E+1] exclusive prefix sum of counts
    row2slot: np.ndarray  # [N*k] grouped row -> flat slot t*k + j
    row2tok: np.ndarray   # [N*k] grouped row -> token t
    slot2row: np.ndarray  # [N*k] flat slot -> grouped row


def group_by_expert(idx, E: int = EXPERTS) -> Grouping:
    """Group the (token, slot) pairs by expert, token-major inside an expert.

    Guide, "What to verify in a deployment": the expert path groups tokens by
    expert.  A stable sort of the flat slot list by expert id: rows of
    expert e are contiguous, in increasing token order.
    """
    idx = np.asarray(idx)
    k = idx.shape[1]
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    row2slot = np.argsort(flat, kind="stable").astype(np.int64)
    slot2row = np.empty_like(row2slot)
    slot2row[row2slot] = np.arange(row2slot.shape[0])
    return Grouping(counts=counts, offsets=offsets, row2slot=row2slot,
                    row2tok=row2slot // k, slot2row=slot2row)


def expert_hidden(Xe, W_gate_e, W_up_e) -> np.ndarray:
    """H = silu(Xe W_gate^T) * (Xe W_up^T): the gated SiLU half of an expert."""
    Xe = f64(Xe)
    G = Xe @ f64(W_gate_e).T
    U = Xe @ f64(W_up_e).T
    return silu(G) * U


def expert_forward(Xe, W_gate_e, W_up_e, W_down_e) -> np.ndarray:
    """One expert: W_down (silu(W_gate x) * (W_up x)), 2048 -> 1536 -> 2048."""
    return expert_hidden(Xe, W_gate_e, W_up_e) @ f64(W_down_e).T


@dataclass
class LayerResult:
    out: np.ndarray        # [N, d] layer output
    routing: Routing | None
    grouping: Grouping
    H: np.ndarray          # [N*k, ff] expert hidden rows, grouped order
    Y: np.ndarray          # [N*k, d] expert output rows, grouped order


def moe_apply(X, idx, w, W_gate, W_up, W_down, routing: Routing | None = None) -> LayerResult:
    """Expert evaluation and weighted combine for given routing decisions.

    Groups slots by expert, runs every non-empty expert once on its rows and
    accumulates out[t] = sum_j w[t, j] * Y[row of (t, j)].
    """
    X = f64(X)
    idx = np.asarray(idx)
    w = f64(w)
    N, k = idx.shape
    E = W_gate.shape[0]
    d = W_down.shape[1]
    ff = W_gate.shape[1]
    g = group_by_expert(idx, E)
    H = np.zeros((N * k, ff))
    Y = np.zeros((N * k, d))
    for e in range(E):
        a, b = int(g.offsets[e]), int(g.offsets[e + 1])
        if a == b:
            continue
        Xe = X[g.row2tok[a:b]]
        H[a:b] = expert_hidden(Xe, W_gate[e], W_up[e])
        Y[a:b] = H[a:b] @ f64(W_down[e]).T
    out = np.zeros((N, d))
    for j in range(k):
        out += w[:, j:j + 1] * Y[g.slot2row.reshape(N, k)[:, j]]
    return LayerResult(out=out, routing=routing, grouping=g, H=H, Y=Y)


def moe_forward(X, W_r, bias, W_gate, W_up, W_down, k: int = TOP_K) -> LayerResult:
    """The whole sparse feed-forward layer on normalised hidden states X."""
    r = route(X, W_r, bias, k=k)
    return moe_apply(X, r.idx, r.w, W_gate, W_up, W_down, routing=r)


def dense_masked_forward(X, W_r, bias, W_gate, W_up, W_down, k: int = TOP_K) -> np.ndarray:
    """Brute force: every expert on every token, combined through a 0/w mask.

    Equal to moe_forward in exact arithmetic; used to pin the grouping and
    combine steps.
    """
    X = f64(X)
    r = route(X, W_r, bias, k=k)
    N = X.shape[0]
    E = W_gate.shape[0]
    mask = np.zeros((N, E))
    np.put_along_axis(mask, r.idx, r.w, axis=1)
    out = np.zeros((N, W_down.shape[1]))
    for e in range(E):
        out += mask[:, e:e + 1] * expert_forward(X, W_gate[e], W_up[e], W_down[e])
    return out


def block_input(x) -> np.ndarray:
    """MoE input of a block: RMSNorm of the fp32 residual stream, stored as bf16."""
    return round_bf16(rmsnorm(x))


def block_forward(x, W_r, bias, W_gate, W_up, W_down) -> np.ndarray:
    """One block's feed-forward half: x + MoE(bf16(RMSNorm(x))).

    Guide, "The exact checkpoint": normalise, run the feed-forward network,
    add the residual.  The bf16 rounding of the MoE input is the layer's
    input dtype contract (activations enter the layer as bf16).
    """
    x = f64(x)
    return x + moe_forward(block_input(x), W_r, bias, W_gate, W_up, W_down).out
