"""lfm_moe_forward_noalloc (the allocation-free layer entry point) through
the C ABI, against lfm_moe_forward on the same inputs: bit for bit, on
three calls in a row, each with a smaller batch (256 and 64 tokens on the
grouped kernels, 3 on the weight-streaming kernels), and with no change of
the device's free memory."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import cached_layer
from parity import device_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import biased_sigmoid_top_amd as m
    return m


def _call(lib, fn, X, dev, out, N):
    st = getattr(lib, fn)(X.data_ptr(), dev["W_r"].data_ptr(), dev["bias"].data_ptr(),
                          dev["W_gateup"].data_ptr(), dev["W_down"].data_ptr(), out.data_ptr(), N,
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, (fn, st, lib.lfm_moe_last_error())


def test_noalloc_forward_equals_forward(moe):
    from biased_sigmoid_top_amd import _lib
    lib = _lib.load()
    w = synth.WORKLOADS["tiny_n32"]
    dev = device_weights(cached_layer(w["N"], w["seed"], w["skew"]))
    cases = []
    for N, seed in ((_lib.NOALLOC_MAX_TOKENS, 1900), (64, 1901), (3, 1902)):
        X = torch.from_numpy(oracle.block_input(synth.hidden_states(N, seed).numpy())).to(torch.bfloat16).cuda()
        cases.append((N, X, torch.full((N, 2048), np.nan, device="cuda"),
                      torch.full((N, 2048), np.nan, device="cuda")))
    # lfm_moe_forward first (its own workspace allocated here), and one
    # allocation-free call, whose first use on the device loads the
    # library's code object with the static array; then the device's free
    # memory must stay as it is over the two measured calls.
    for N, X, _, want in cases:
        print(f"[gpu] lfm_moe_forward N={N}", flush=True)
        _call(lib, "lfm_moe_forward", X, dev, want, N)
    N, X, got, _ = cases[1]
    _call(lib, "lfm_moe_forward_noalloc", X, dev, got, N)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for N, X, got, _ in cases:
        got.fill_(np.nan)
    for N, X, got, _ in cases:
        print(f"[gpu] lfm_moe_forward_noalloc N={N}", flush=True)
        _call(lib, "lfm_moe_forward_noalloc", X, dev, got, N)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0, "device memory changed during the allocation-free calls"
    for N, X, got, want in cases:
        assert torch.isfinite(got).all().item()
        assert torch.equal(got, want), f"N={N}: allocation-free result differs from lfm_moe_forward"
    # Past the limit: an error before any launch, and the next call still works.
    N = _lib.NOALLOC_MAX_TOKENS + 1
    X = torch.zeros(N, 2048, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(N, 2048, device="cuda")
    st = lib.lfm_moe_forward_noalloc(X.data_ptr(), dev["W_r"].data_ptr(), dev["bias"].data_ptr(),
                                     dev["W_gateup"].data_ptr(), dev["W_down"].data_ptr(), out.data_ptr(), N,
                                     None)
    assert st == _lib.ERR_INVALID_ARGUMENT and b"NOALLOC_MAX_TOKENS" in lib.lfm_moe_last_error()
    N, X, got, want = cases[1]
    got.fill_(np.nan)
    _call(lib, "lfm_moe_forward_noalloc", X, dev, got, N)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
