"""Seeded synthetic inputs for the MoE layer workloads.

Shared by the tests, the bench and the smoke check, on both sides of every
parity comparison.  It only draws random numbers, scales them to the stated
distributions and rounds them to their storage dtypes; it holds none of the
layer's arithmetic (no normalisation, routing or expert math).

Recipe (CPU torch.Generator, fixed draw order):

* generator ``seed``: z [N, 2048] fp32 ~ N(0, 1) (the pre-normalisation
  hidden states), then W_r [64, 2048] = bf16(0.02 * N(0, 1)), then
  bias [64] fp32 ~ U(-0.25, 0.25) (plus 0.5 on experts 0..7 when ``skew``).
* expert e uses its own generator, seeded ``expert_seed(seed, e)``:
  W_gate [1536, 2048], W_up [1536, 2048], W_down [2048, 1536], each
  bf16(0.02 * N(0, 1)), drawn in that order.  Per-expert streams let a
  checker regenerate only the experts it needs.
* a stack of blocks: the residual stream x0 [N, 2048] fp32 ~ N(0, 1) from
  generator ``seed``; block l's router, bias and experts are a layer drawn
  with seed ``block_seed(seed, l)`` (no z).
"""

from __future__ import annotations

import hashlib

import torch

HIDDEN = 2048
EXPERTS = 64
FF = 1536
WEIGHT_STD = 0.02
BIAS_HALF_RANGE = 0.25
SKEW_EXPERTS = 8
SKEW_BOOST = 0.5


def expert_seed(seed: int, e: int) -> int:
    return seed * 1_000_003 + 1 + e


def block_seed(seed: int, block: int) -> int:
    return seed * 1000 + block


def _normal(shape, g, std=1.0):
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    return t * std if std != 1.0 else t


def hidden_states(N: int, seed: int, d: int = HIDDEN) -> torch.Tensor:
    """z [N, d] fp32 ~ N(0, 1): the first draw of generator ``seed``."""
    g = torch.Generator().manual_seed(seed)
    return _normal((N, d), g)


def router_params(seed: int, N_skip: int, skew: bool = False, d: int = HIDDEN,
                  E: int = EXPERTS):
    """W_r bf16 [E, d] and bias fp32 [E], drawn after ``N_skip`` rows of z."""
    g = torch.Generator().manual_seed(seed)
    if N_skip:
        _normal((N_skip, d), g)
    W_r = _normal((E, d), g, WEIGHT_STD).bfloat16()
    bias = torch.rand(E, generator=g, dtype=torch.float32) * (2 * BIAS_HALF_RANGE) - BIAS_HALF_RANGE
    if skew:
        bias[:SKEW_EXPERTS] += SKEW_BOOST
    return W_r, bias


def expert_params(seed: int, e: int, d: int = HIDDEN, ff: int = FF):
    """(W_gate [ff, d], W_up [ff, d], W_down [d, ff]) bf16 of expert e."""
    g = torch.Generator().manual_seed(expert_seed(seed, e))
    W_gate = _normal((ff, d), g, WEIGHT_STD).bfloat16()
    W_up = _normal((ff, d), g, WEIGHT_STD).bfloat16()
    W_down = _normal((d, ff), g, WEIGHT_STD).bfloat16()
    return W_gate, W_up, W_down


def layer_params(seed: int, N_skip: int = 0, skew: bool = False, d: int = HIDDEN,
                 E: int = EXPERTS, ff: int = FF) -> dict:
    """Router, bias and all experts of one layer (CPU tensors)."""
    W_r, bias = router_params(seed, N_skip, skew, d, E)
    W_gate = torch.empty(E, ff, d, dtype=torch.bfloat16)
    W_up = torch.empty(E, ff, d, dtype=torch.bfloat16)
    W_down = torch.empty(E, d, ff, dtype=torch.bfloat16)
    for e in range(E):
        W_gate[e], W_up[e], W_down[e] = expert_params(seed, e, d, ff)
    return dict(W_r=W_r, bias=bias, W_gate=W_gate, W_up=W_up, W_down=W_down)


def layer_inputs(N: int, seed: int, skew: bool = False, d: int = HIDDEN,
                 E: int = EXPERTS, ff: int = FF) -> dict:
    """z plus all parameters of one single-layer workload."""
    z = hidden_states(N, seed, d)
    p = layer_params(seed, N_skip=N, skew=skew, d=d, E=E, ff=ff)
    p["z"] = z
    return p


def stack_residual(N: int, seed: int, d: int = HIDDEN) -> torch.Tensor:
    """x0 [N, d] fp32 ~ N(0, 1) of a block stack."""
    return hidden_states(N, seed, d)


def stack_block_params(seed: int, block: int, d: int = HIDDEN, E: int = EXPERTS,
                       ff: int = FF) -> dict:
    return layer_params(block_seed(seed, block), 0, False, d, E, ff)


# Verification-shaped batches of speculative decoding (orcarouter.ai page
# "LFM2.5-24B-A2B-DSpark ist live auf Hugging Face", sections "Was ist
# eigentlich im Repository?" and "Es ausführen": the drafter proposes blocks
# of 9 and the target verifies ten tokens per request per step; verifying k
# tokens activates more experts than decoding one).  c concurrent requests
# make a batch of 10c tokens.  One layer, drawn with seed 5 for the largest
# batch, serves the whole series: the batch of c requests is the first 10c
# rows of its z, so the growth of the active-expert set is seen on one model.
VERIFY = dict(seed=5, tokens_per_request=10, concurrency=(1, 2, 4, 8, 16, 32, 64))


def verify_batch_sizes() -> list:
    return [VERIFY["tokens_per_request"] * c for c in VERIFY["concurrency"]]


def verify_inputs() -> dict:
    """z for the largest verification batch plus the layer's parameters."""
    return layer_inputs(max(verify_batch_sizes()), VERIFY["seed"])


# The single-layer workloads: (name, N, seed, skew).
WORKLOADS = {
    "tiny_n32": dict(N=32, seed=0, skew=False),
    "decode_n64": dict(N=64, seed=1, skew=False),
    "prefill_n4096": dict(N=4096, seed=2, skew=False),
    "skewed_n16384": dict(N=16384, seed=3, skew=True),
}
STACK = dict(N=512, seed=4, blocks=38)


def sha256(t: torch.Tensor) -> str:
    """Digest of a tensor's bytes, recorded beside measurements."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return hashlib.sha256(t.numpy().tobytes()).hexdigest()
