"""The expert path on caller-given routing (lfm_moe_experts_ws and
lfm_moe_experts_fp8_ws) on the MI355X, through the C ABI.

* On the layer's own routing it reproduces lfm_moe_forward_ws /
  lfm_moe_forward_fp8_ws bit for bit (decode-shaped and grouped batches).
* On the oracle's routing it meets the layer's bar on every token, near
  ties included: with the selection held fixed there is no token to set
  aside.
* Selections outside [0, 64) or repeated within a token are replaced by the
  documented rule (its host mirror is pinned in test_abi.py) and the call
  then equals a call on the replaced selections.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import cached_layer
from parity import (check_out, device_inputs, fp8_output_check, oracle_fp8_experts, oracle_inputs,
                    sanitize_routing)

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


def _case(moe):
    """Oracle inputs and device weights (bf16 packed and FP8) of the decode workload's layer."""
    if "case" not in _STATE:
        w = synth.WORKLOADS["decode_n64"]
        layer = cached_layer(w["N"], w["seed"], w["skew"])
        inp = oracle_inputs(layer)
        dev = device_inputs(layer, inp["X"])
        _step("pack_fp8_gateup / pack_fp8_down")
        dev["gateup_fp8"] = moe.pack_fp8_gateup(layer["W_gate"].cuda(), layer["W_up"].cuda())
        dev["down_fp8"] = moe.pack_fp8_down(layer["W_down"].cuda())
        torch.cuda.synchronize()
        _STATE["case"] = (inp, dev)
    return _STATE["case"]


def _x(N, seed):
    X = oracle.block_input(synth.hidden_states(N, seed).numpy())
    return X, torch.from_numpy(X).to(torch.bfloat16).cuda()


def _experts(moe, dev, fp8, X, idx, w, ws):
    if fp8:
        return moe.experts_fp8(X, idx, w, dev["gateup_fp8"], dev["down_fp8"], workspace=ws)
    return moe.experts(X, idx, w, dev["W_gateup"], dev["W_down"], workspace=ws)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("N", [3, 64, 700, 5000])
def test_experts_equal_the_layer_on_its_own_routing(moe, N, fp8):
    """N = 5000 ends in a partial 16-token histogram block."""
    from biased_sigmoid_top_amd import _lib
    inp, dev = _case(moe)
    _, X = _x(N, 2100 + N)
    ws = moe.alloc_workspace(N)
    _step(f"forward{'_fp8' if fp8 else ''}_ws N={N}")
    if fp8:
        out_f = moe.forward_fp8(X, dev["W_r"], dev["bias"], dev["gateup_fp8"], dev["down_fp8"], workspace=ws)
    else:
        out_f = moe.forward(X, dev["W_r"], dev["bias"], dev["W_gateup"], dev["W_down"], workspace=ws)
    idx = moe.workspace_view(ws, N, _lib.WS_IDX, torch.int32, (N, 4)).clone()
    w = moe.workspace_view(ws, N, _lib.WS_W, torch.float32, (N, 4)).clone()
    ws2 = moe.alloc_workspace(N)
    ws2.fill_(0xFF)
    _step(f"experts{'_fp8' if fp8 else ''}_ws N={N}")
    out_e = _experts(moe, dev, fp8, X, idx, w, ws2)
    torch.cuda.synchronize()
    assert torch.equal(out_e, out_f), "the expert path differs from the layer on the layer's routing"
    assert torch.equal(moe.workspace_view(ws2, N, _lib.WS_IDX, torch.int32, (N, 4)), idx)
    assert torch.equal(moe.workspace_view(ws2, N, _lib.WS_W, torch.float32, (N, 4)), w)


@pytest.mark.parametrize("N", [64, 700])
def test_experts_on_the_oracle_routing(moe, N):
    """bf16 experts against oracle.moe_apply on the oracle's own selections and
    weights (the weights handed over in fp32), every token."""
    inp, dev = _case(moe)
    Xo, X = _x(N, 2300 + N)
    r = oracle.route(Xo, inp["W_r"], inp["bias"])
    w32 = r.w.astype(np.float32)
    idx = torch.from_numpy(np.ascontiguousarray(r.idx, dtype=np.int32)).cuda()
    w = torch.from_numpy(w32).cuda()
    _step(f"experts_ws on oracle routing N={N}")
    out = _np(moe.experts(X, idx, w, dev["W_gateup"], dev["W_down"]))
    expect = oracle.moe_apply(Xo, r.idx, w32.astype(np.float64), inp["W_gate"], inp["W_up"],
                              inp["W_down"]).out
    ratio = check_out(out, expect)
    near = int(np.sum(r.margin <= 1e-4))
    print(f"  max|err|/RMS {ratio:.4f} over all {N} tokens ({near} near ties)", flush=True)


@pytest.mark.parametrize("N", [64, 700])
def test_experts_fp8_on_the_oracle_routing(moe, N):
    """FP8 experts against oracle.fp8 on the oracle's routing (the bar of
    parity.fp8_output_check)."""
    from biased_sigmoid_top_amd import _lib
    inp, dev = _case(moe)
    if "q" not in _STATE:
        print("[fp8] oracle block quantisation of 64 x 3 expert matrices", flush=True)
        _STATE["q"] = oracle_fp8_experts(inp)
    q = _STATE["q"]
    Xo, X = _x(N, 2500 + N)
    r = oracle.route(Xo, inp["W_r"], inp["bias"])
    w32 = r.w.astype(np.float32)
    idx = torch.from_numpy(np.ascontiguousarray(r.idx, dtype=np.int32)).cuda()
    w = torch.from_numpy(w32).cuda()
    _step(f"experts_fp8_ws on oracle routing N={N}")
    ws = moe.alloc_workspace(N)
    out = _np(moe.experts_fp8(X, idx, w, dev["gateup_fp8"], dev["down_fp8"], workspace=ws)).astype(np.float64)
    H = _np(moe.workspace_view(ws, N, _lib.WS_H, torch.bfloat16, (4 * N, 1536)).float()).astype(np.float64)
    res = fp8_output_check(out, r.idx, w32.astype(np.float64), H, Xo, q)
    print(f"  all {N} tokens: out vs FP8 oracle on the GPU's H {res['same_codes']:.2e}, end to end "
          f"{res['end_to_end']:.4f} ({res['code_flips']} H codes and {res['scale_flips']} group scales differ)",
          flush=True)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("N", [37, 300])
def test_invalid_routing_is_replaced_by_the_documented_rule(moe, N, fp8):
    from biased_sigmoid_top_amd import _lib
    inp, dev = _case(moe)
    _, X = _x(N, 2700 + N)
    rng = np.random.default_rng(N)
    given = rng.integers(-70, 130, size=(N, 4)).astype(np.int32)
    given[::3, 1] = given[::3, 0]          # a repeat
    given[::5] = given[::5, :1]            # all four the same
    given[1::7, 3] = given[1::7, 2] + 64   # the same id modulo 64
    w = torch.from_numpy(rng.random((N, 4), dtype=np.float32)).cuda()
    want = sanitize_routing(given)
    ws = moe.alloc_workspace(N)
    _step(f"experts{'_fp8' if fp8 else ''}_ws on invalid routing N={N}")
    out = _experts(moe, dev, fp8, X, torch.from_numpy(given).cuda(), w, ws)
    used = _np(moe.workspace_view(ws, N, _lib.WS_IDX, torch.int32, (N, 4)))
    np.testing.assert_array_equal(used, want)
    _step(f"experts{'_fp8' if fp8 else ''}_ws on the replaced routing N={N}")
    out2 = _experts(moe, dev, fp8, X, torch.from_numpy(want).cuda(), w, moe.alloc_workspace(N))
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert torch.isfinite(out).all().item()


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("N", [64, 700])
def test_experts_graph_replays_match_eager(moe, N, fp8):
    """The expert path records no allocation, memset or host synchronisation
    either: captured in a HIP graph, three replays (with eager calls and
    synchronisations between them) equal the eager result bit for bit."""
    inp, dev = _case(moe)
    _, X = _x(N, 2900 + N)
    idx = torch.from_numpy(np.stack([np.random.default_rng(N).choice(64, 4, replace=False)
                                     for _ in range(N)]).astype(np.int32)).cuda()
    w = torch.full((N, 4), 0.25, device="cuda")
    ws = moe.alloc_workspace(N)
    _step(f"graph capture experts{'_fp8' if fp8 else ''}_ws N={N}")
    eager = _experts(moe, dev, fp8, X, idx, w, ws).clone()

    def run(out):
        if fp8:
            moe.experts_fp8(X, idx, w, dev["gateup_fp8"], dev["down_fp8"], out=out, workspace=ws)
        else:
            moe.experts(X, idx, w, dev["W_gateup"], dev["W_down"], out=out, workspace=ws)

    out = torch.empty_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(out)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out)
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager call"
        run(torch.empty_like(eager))
        torch.cuda.synchronize()


def test_experts_with_no_tokens_is_a_no_op(moe):
    _, dev = _case(moe)
    X = torch.empty(0, 2048, dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(0, 4, dtype=torch.int32, device="cuda")
    w = torch.empty(0, 4, dtype=torch.float32, device="cuda")
    assert moe.experts(X, idx, w, dev["W_gateup"], dev["W_down"]).shape == (0, 2048)
    assert moe.experts_fp8(X, idx, w, dev["gateup_fp8"], dev["down_fp8"]).shape == (0, 2048)
