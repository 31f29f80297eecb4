"""The stage entry points (lfm_moe_stage_dispatch, _gateup, _down, _combine)
on the MI355X, through the C ABI.

* Chained on one workspace they equal lfm_moe_experts_ws bit for bit, on the
  streaming path (64 tokens) and the grouped path (700 tokens).
* Each stage alone against the oracle, on inputs that the oracle supplies:
  the grouping of the oracle's selections equals oracle.group_by_expert; H
  from gate/up is within half a bf16 ulp (plus the fp32 accumulation error)
  of the oracle's; Y from the oracle's bf16-rounded H (written into the H
  region) matches that H times W_down in float64 to fp32 accumulation
  error; out from the oracle's Y (written into the Y region) matches the
  float64 weighted sum to fp32 rounding.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import cached_layer
from parity import device_weights, oracle_inputs

pytestmark = pytest.mark.gpu

_STATE = {}


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import biased_sigmoid_top_amd as m
    return m


def _step(msg):
    print(f"[gpu] {msg}", flush=True)


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _case():
    """Oracle arrays and device weights of the 64-token decode workload's layer."""
    if "case" not in _STATE:
        w = synth.WORKLOADS["decode_n64"]
        layer = cached_layer(w["N"], w["seed"], w["skew"])
        _STATE["case"] = (oracle_inputs(layer), device_weights(layer))
    return _STATE["case"]


def _x(N, seed):
    X = oracle.block_input(synth.hidden_states(N, seed).numpy())
    return X, torch.from_numpy(X).to(torch.bfloat16).cuda()


def _chain(moe, dev, X, idx, w, ws):
    moe.stage_dispatch(idx, w, ws)
    moe.stage_gateup(X, dev["W_gateup"], ws)
    moe.stage_down(dev["W_down"], X.shape[0], ws)
    return moe.stage_combine(X.shape[0], ws)


@pytest.mark.parametrize("N", [3, 64, 700])
def test_stage_chain_equals_the_expert_path(moe, N):
    inp, dev = _case()
    _, X = _x(N, 4100 + N)
    rng = np.random.default_rng(N)
    idx = torch.from_numpy(np.stack([rng.choice(64, 4, replace=False) for _ in range(N)]).astype(np.int32)).cuda()
    w = torch.from_numpy(rng.random((N, 4), dtype=np.float32)).cuda()
    ws = moe.alloc_workspace(N)
    ws.fill_(0xFF)
    _step(f"stage chain N={N}")
    out = _chain(moe, dev, X, idx, w, ws)
    _step(f"experts_ws N={N}")
    ref = moe.experts(X, idx, w, dev["W_gateup"], dev["W_down"], workspace=moe.alloc_workspace(N))
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "the stage chain differs from lfm_moe_experts_ws"


@pytest.mark.parametrize("N", [3, 64, 700])
def test_each_stage_against_the_oracle(moe, N):
    from biased_sigmoid_top_amd import _lib
    inp, dev = _case()
    Xo, X = _x(N, 4300 + N)
    r = oracle.route(Xo, inp["W_r"], inp["bias"])
    w32 = r.w.astype(np.float32)
    ws = moe.alloc_workspace(N)
    ws.fill_(0xFF)
    view = lambda reg, dt, shape: moe.workspace_view(ws, N, reg, dt, shape)

    _step(f"stage_dispatch on the oracle's routing N={N}")
    moe.stage_dispatch(torch.from_numpy(np.ascontiguousarray(r.idx, dtype=np.int32)).cuda(),
                       torch.from_numpy(w32).cuda(), ws)
    g = oracle.group_by_expert(r.idx)
    np.testing.assert_array_equal(_np(view(_lib.WS_OFFSETS, torch.int32, (65,))), g.offsets)
    np.testing.assert_array_equal(_np(view(_lib.WS_ROW2SLOT, torch.int32, (4 * N,))), g.row2slot)
    np.testing.assert_array_equal(_np(view(_lib.WS_W, torch.float32, (N, 4))), w32)

    ref = oracle.moe_apply(Xo, r.idx, w32.astype(np.float64), inp["W_gate"], inp["W_up"], inp["W_down"])
    H_ref = np.empty_like(ref.H)
    H_ref[g.row2slot] = ref.H
    Y_ref = np.empty_like(ref.Y)
    Y_ref[g.row2slot] = ref.Y

    _step(f"stage_gateup N={N}")
    moe.stage_gateup(X, dev["W_gateup"], ws)
    H = _np(view(_lib.WS_H, torch.bfloat16, (4 * N, 1536)).float()).astype(np.float64)
    _, ex = np.frexp(H_ref)
    h_rms = np.sqrt(np.mean(H_ref ** 2))
    assert np.all(np.abs(H - H_ref) <= np.ldexp(1.0, ex - 9) * (1 + 2 ** -6) + 1e-4 * h_rms)

    _step(f"stage_down on the oracle's H N={N}")
    Hq = oracle.round_bf16(H_ref)
    view(_lib.WS_H, torch.bfloat16, (4 * N, 1536)).copy_(torch.from_numpy(Hq).to(torch.bfloat16))
    moe.stage_down(dev["W_down"], N, ws)
    Y = _np(view(_lib.WS_Y, torch.float32, (4 * N, 2048))).astype(np.float64)
    Yq = np.zeros_like(Y_ref)
    flat = r.idx.reshape(-1)
    for e in np.unique(flat):
        rows = np.nonzero(flat == e)[0]
        Yq[rows] = Hq[rows] @ inp["W_down"][e].astype(np.float64).T
    y_rms = np.sqrt(np.mean(Yq ** 2))
    err = np.max(np.abs(Y - Yq)) / y_rms
    print(f"  down on the oracle's H: max|Y - Y_oracle| / RMS = {err:.2e}", flush=True)
    assert err <= 1e-4

    _step(f"stage_combine on the oracle's Y N={N}")
    Y32 = Y_ref.astype(np.float32)
    view(_lib.WS_Y, torch.float32, (4 * N, 2048)).copy_(torch.from_numpy(Y32))
    resid = torch.from_numpy(synth.hidden_states(N, 4500 + N).numpy().astype(np.float32)).cuda()
    out = _np(moe.stage_combine(N, ws)).astype(np.float64)
    out_r = _np(moe.stage_combine(N, ws, resid=resid)).astype(np.float64)
    expect = (w32.astype(np.float64)[:, :, None] * Y32.astype(np.float64).reshape(N, 4, -1)).sum(axis=1)
    o_rms = np.sqrt(np.mean(expect ** 2))
    assert np.max(np.abs(out - expect)) <= 1e-5 * o_rms
    expect_r = _np(resid).astype(np.float64) + expect
    assert np.max(np.abs(out_r - expect_r)) <= 1e-5 * np.sqrt(np.mean(expect_r ** 2))
