"""The C ABI library loads, exports what include/lfm_moe.h declares, and
rejects bad arguments before any HIP call (so these run without a GPU)."""

import ctypes
import re

import numpy as np

import pytest

from biased_sigmoid_top_amd import _lib

FAKE = 1 << 40  # aligned host-side stand-in addresses: never dereferenced here


def _addr(i):
    return FAKE + i * (1 << 34)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_function_is_exported(lib):
    names = _lib.declared_functions()
    assert len(names) == len(_lib.SIGNATURES)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing
    assert set(names) == set(_lib.SIGNATURES)


def test_abi_version_matches_header(lib):
    with open(_lib.HEADER) as f:
        v = int(re.search(r"#define LFM_MOE_ABI_VERSION (\d+)", f.read()).group(1))
    assert lib.lfm_moe_abi_version() == v


def test_workspace_layout(lib):
    for N in [1, 16, 17, 64, 255, 256, 257, 4096, 16384]:
        total = lib.lfm_moe_workspace_bytes(N)
        offs = [lib.lfm_moe_workspace_offset(N, r) for r in range(13)] + [total]
        assert offs[0] == 0
        assert all(o % 256 == 0 for o in offs)
        assert offs == sorted(offs)
        size = lambda r: offs[r + 1] - offs[r]
        # H and Y regions hold 4N rows.
        assert size(_lib.WS_H) >= 4 * N * 1536 * 2
        assert size(_lib.WS_Y) >= 4 * N * 2048 * 4
        assert size(_lib.WS_X) >= N * 2048 * 2
        if N <= 2048:
            assert size(_lib.WS_ROUTER_PARTIAL) >= -(-N // 16) * 16 * 16 * 64 * 4
        else:
            assert size(_lib.WS_ROUTER_PARTIAL) == 0  # the fused router keeps its partials in LDS
        # Quantised rows and scales of the FP8 layer's grouped path (above 256 tokens only).
        fp8 = N > _lib.FP8_STREAM_TOKENS
        assert size(_lib.WS_XQ) >= (N * 2048 if fp8 else 0)
        assert size(_lib.WS_XS) >= (N * 16 * 4 if fp8 else 0)
        assert size(_lib.WS_HQ) >= (4 * N * 1536 if fp8 else 0)
        assert size(_lib.WS_HS) >= (4 * N * 12 * 4 if fp8 else 0)
        if not fp8:
            assert all(size(r) == 0 for r in (_lib.WS_XQ, _lib.WS_XS, _lib.WS_HQ, _lib.WS_HS))
    assert lib.lfm_moe_workspace_bytes(-1) == 0
    assert lib.lfm_moe_workspace_offset(10, 99) == ctypes.c_size_t(-1).value


def _fwd(lib, X, Wr, b, Wgu, Wd, out, N):
    return lib.lfm_moe_forward(X, Wr, b, Wgu, Wd, out, N, None)


def test_forward_argument_checks(lib):
    a = [_addr(i) for i in range(6)]
    assert _fwd(lib, *a, 0) == _lib.OK  # N == 0: nothing launched
    assert _fwd(lib, *a, -1) == _lib.ERR_INVALID_ARGUMENT
    assert _fwd(lib, *a, (1 << 24) + 1) == _lib.ERR_INVALID_ARGUMENT
    for i in range(6):
        b = list(a)
        b[i] = None
        assert _fwd(lib, *b, 8) == _lib.ERR_INVALID_ARGUMENT
        assert b"null" in lib.lfm_moe_last_error()
        b = list(a)
        b[i] = a[i] + 4
        assert _fwd(lib, *b, 8) == _lib.ERR_INVALID_ARGUMENT
        assert b"aligned" in lib.lfm_moe_last_error()
    # Output overlapping an input.
    b = list(a)
    b[5] = a[0] + 1024
    assert _fwd(lib, *b, 8) == _lib.ERR_INVALID_ARGUMENT
    b = list(a)
    b[5] = a[3] + 4096
    assert _fwd(lib, *b, 8) == _lib.ERR_INVALID_ARGUMENT


def test_forward_ws_checks(lib):
    a = [_addr(i) for i in range(6)]
    need = lib.lfm_moe_workspace_bytes(100)
    ws = _addr(7)
    f = lib.lfm_moe_forward_ws
    assert f(*a, 100, ws, need - 1, None) == _lib.ERR_WORKSPACE_TOO_SMALL
    assert f(*a, 100, None, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert f(*a, 100, ws + 16, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert f(*a, 100, a[5], need, None) == _lib.ERR_INVALID_ARGUMENT  # overlaps out
    for i in range(5):                                 # starts 256 bytes before an input
        assert f(*a, 100, a[i] - 256, need, None) == _lib.ERR_INVALID_ARGUMENT
        assert b"workspace overlaps an input" in lib.lfm_moe_last_error()
    blk = lib.lfm_moe_block_forward_ws
    assert blk(a[0], a[1], a[2], a[3], a[4], 100, a[3] + 4096, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert b"workspace overlaps an input" in lib.lfm_moe_last_error()
    assert f(*a, 0, None, 0, None) == _lib.OK


def test_route_rmsnorm_block_checks(lib):
    a = [_addr(i) for i in range(5)]
    assert lib.lfm_moe_route(*a, 0, None) == _lib.OK
    assert lib.lfm_moe_route(*a, -3, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_route(a[0], None, a[2], a[3], a[4], 4, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_route(a[0], a[1], a[2], a[3], a[3] + 16, 4, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_rmsnorm(a[0], a[1], 0, None) == _lib.OK
    assert lib.lfm_moe_rmsnorm(a[0], a[0] + 64, 4, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_rmsnorm(None, a[1], 4, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_block_forward(a[0], a[1], a[2], a[3], a[4], 0, None) == _lib.OK
    assert lib.lfm_moe_block_forward(a[0], a[1], a[2], a[3], None, 4, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_block_forward_ws(a[0], a[1], a[2], a[3], a[4], 4, None, 0, None) == _lib.ERR_INVALID_ARGUMENT


def test_stack_forward_checks(lib):
    """lfm_moe_stack_forward_ws checks every block before launching anything
    (each call here fails or is a no-op before any HIP call)."""
    import ctypes
    a = [_addr(i) for i in range(5)]
    need = lib.lfm_moe_workspace_bytes(100)
    ws = _addr(7)
    good = _lib.BlockWeights(a[1], a[2], a[3], a[4])
    blocks = (_lib.BlockWeights * 3)(good, good, _lib.BlockWeights(a[1], a[2], a[3], None))
    f = lib.lfm_moe_stack_forward_ws
    p = ctypes.addressof(blocks)
    assert f(a[0], p, 3, 100, ws, need, None) == _lib.ERR_INVALID_ARGUMENT  # block 2 has no W_down
    assert b"null tensor pointer" in lib.lfm_moe_last_error()
    assert f(a[0], p, -1, 100, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert f(a[0], None, 2, 100, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert f(a[0], p, 2, 100, ws, need - 1, None) == _lib.ERR_WORKSPACE_TOO_SMALL
    assert f(a[0], p, 2, 100, a[3] + 4096, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert b"workspace overlaps an input" in lib.lfm_moe_last_error()
    assert f(a[0], p, 3, 0, None, 0, None) == _lib.OK   # N == 0
    assert f(a[0], p, 0, 100, ws, need, None) == _lib.OK  # no blocks
    assert f(a[0], None, 0, 100, None, 0, None) == _lib.OK


def test_stage_checks(lib):
    """The stage entry points check their tensors and the workspace before
    any HIP call."""
    a = [_addr(i) for i in range(5)]
    need = lib.lfm_moe_workspace_bytes(100)
    ws = _addr(7)
    assert lib.lfm_moe_stage_dispatch(a[0], a[1], 100, ws, need - 1, None) == _lib.ERR_WORKSPACE_TOO_SMALL
    assert lib.lfm_moe_stage_dispatch(None, a[1], 100, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_stage_dispatch(a[0], a[1] + 4, 100, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_stage_dispatch(a[0], a[1], -1, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_stage_dispatch(a[0], a[1], 0, None, 0, None) == _lib.OK
    assert lib.lfm_moe_stage_gateup(a[0], a[3], 100, a[3] + 4096, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert b"workspace overlaps an input" in lib.lfm_moe_last_error()
    assert lib.lfm_moe_stage_gateup(a[0], None, 100, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_stage_down(a[4], 100, None, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_stage_down(a[4], 100, ws + 16, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_stage_combine(None, None, 100, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_stage_combine(None, ws + 256, 100, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert b"workspace overlaps the output" in lib.lfm_moe_last_error()
    assert lib.lfm_moe_stage_combine(a[0] + 64, a[0], 100, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_stage_combine(a[0], a[0], 0, None, 0, None) == _lib.OK


def test_route_ws_checks(lib):
    """lfm_moe_route_ws: the router workspace is the partial logits of up to
    2048 tokens (none above), checked like the layer's."""
    # X, W_r, bias, idx, w
    a = [_addr(i) for i in range(5)]
    ws = _addr(7)
    rb = lib.lfm_moe_route_workspace_bytes
    assert rb(64) == 4 * 16 * 16 * 64 * 4 and rb(2048) == 128 * 16 * 16 * 64 * 4
    assert rb(2049) == 0 and rb(16384) == 0 and rb(-1) == 0 and rb(0) == 0
    f = lib.lfm_moe_route_ws
    need = rb(100)
    assert f(*a, 0, None, 0, None) == _lib.OK
    assert f(*a, -1, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert f(*a, 100, None, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert f(*a, 100, ws + 16, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert f(*a, 100, ws, need - 1, None) == _lib.ERR_WORKSPACE_TOO_SMALL
    for i in range(5):                                   # workspace over any tensor argument
        assert f(*a, 100, a[i] - 256, need, None) == _lib.ERR_INVALID_ARGUMENT
        assert b"workspace overlaps" in lib.lfm_moe_last_error()
    b = list(a)
    b[3] = a[0] + 64                                     # selections written over X
    assert f(*b, 100, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_route(*b, 100, None) == _lib.ERR_INVALID_ARGUMENT
    # Above 2048 tokens no workspace is needed, so none is checked.
    for i in range(5):
        c = list(a)
        c[i] = None
        assert f(*c, 4096, None, 0, None) == _lib.ERR_INVALID_ARGUMENT


def test_noalloc_forward_checks(lib):
    """lfm_moe_forward_noalloc rejects a batch past its static workspace
    before any HIP call, checks its tensors like lfm_moe_forward, and its
    array holds the workspace of the largest batch it takes."""
    a = [_addr(i) for i in range(6)]
    f = lib.lfm_moe_forward_noalloc
    assert lib.lfm_moe_workspace_bytes(_lib.NOALLOC_MAX_TOKENS) <= _lib.NOALLOC_SCRATCH_BYTES
    assert f(*a, 0, None) == _lib.OK
    assert f(*a, _lib.NOALLOC_MAX_TOKENS + 1, None) == _lib.ERR_INVALID_ARGUMENT
    assert b"NOALLOC_MAX_TOKENS" in lib.lfm_moe_last_error()
    assert f(*a, -1, None) == _lib.ERR_INVALID_ARGUMENT
    for i in range(6):
        b = list(a)
        b[i] = None
        assert f(*b, 8, None) == _lib.ERR_INVALID_ARGUMENT
    b = list(a)
    b[5] = a[0] + 1024
    assert f(*b, 8, None) == _lib.ERR_INVALID_ARGUMENT
    with open(_lib.HEADER) as fh:
        text = fh.read()
    assert f"#define LFM_MOE_NOALLOC_MAX_TOKENS {_lib.NOALLOC_MAX_TOKENS}" in text
    assert "#define LFM_MOE_NOALLOC_SCRATCH_BYTES (16u << 20)" in text


def test_pack_checks(lib):
    a = [_addr(i) for i in range(3)]
    assert lib.lfm_moe_pack_gateup(a[0], None, a[2], None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_pack_gateup(a[0], a[1], a[0] + 256, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_pack_gateup(a[0] + 2, a[1], a[2], None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_pack_down(a[0], a[0], None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.lfm_moe_pack_down(None, a[1], None) == _lib.ERR_INVALID_ARGUMENT
    st = lib.lfm_moe_pack_gateup_stacked
    assert st(a[0], None, None) == _lib.ERR_INVALID_ARGUMENT
    assert st(a[0] + 8, a[1], None) == _lib.ERR_INVALID_ARGUMENT
    assert st(a[0], a[0] + 2 * 64 * 3072 * 2048 - 16, None) == _lib.ERR_INVALID_ARGUMENT  # last 16 bytes
    s8 = lib.lfm_moe_pack_fp8_gateup_stacked
    assert s8(a[0], a[1], None, None) == _lib.ERR_INVALID_ARGUMENT
    assert s8(a[0], a[0] + 1024, a[2], None) == _lib.ERR_INVALID_ARGUMENT                  # codes over input
    assert s8(a[0], a[1], a[1] + 256, None) == _lib.ERR_INVALID_ARGUMENT                   # scales over codes


def test_fp8_argument_checks(lib):
    a = [_addr(i) for i in range(8)]
    f = lib.lfm_moe_forward_fp8
    assert f(*a, 0, None) == _lib.OK                      # N == 0: nothing launched
    assert f(*a, -1, None) == _lib.ERR_INVALID_ARGUMENT
    assert f(*a, _lib.FP8_MAX_TOKENS + 1, None) == _lib.ERR_INVALID_ARGUMENT
    assert b"FP8_MAX_TOKENS" in lib.lfm_moe_last_error()
    for i in range(8):
        b = list(a)
        b[i] = None
        assert f(*b, 8, None) == _lib.ERR_INVALID_ARGUMENT
        b = list(a)
        b[i] = a[i] + 4
        assert f(*b, 8, None) == _lib.ERR_INVALID_ARGUMENT
    b = list(a)
    b[7] = a[3] + 1024                                      # out inside the gate/up codes
    assert f(*b, 8, None) == _lib.ERR_INVALID_ARGUMENT
    fw = lib.lfm_moe_forward_fp8_ws
    need = lib.lfm_moe_workspace_bytes(8)
    ws = _addr(9)
    assert fw(*a, 0, None, 0, None) == _lib.OK
    assert fw(*a, 8, None, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert fw(*a, 8, ws + 16, need, None) == _lib.ERR_INVALID_ARGUMENT      # not 256-aligned
    assert fw(*a, 8, ws, need - 1, None) == _lib.ERR_WORKSPACE_TOO_SMALL
    assert fw(*a, 8, a[7] - 256, need, None) == _lib.ERR_INVALID_ARGUMENT   # overlaps out
    assert fw(*a, _lib.FP8_MAX_TOKENS + 1, ws, 1 << 40, None) == _lib.ERR_INVALID_ARGUMENT
    for i in range(7):                                      # starts 256 bytes before an input
        assert fw(*a, 8, a[i] - 256, need, None) == _lib.ERR_INVALID_ARGUMENT
        assert b"workspace overlaps an input" in lib.lfm_moe_last_error()
    g, d = lib.lfm_moe_pack_fp8_gateup, lib.lfm_moe_pack_fp8_down
    assert g(a[0], a[1], a[2], None, None) == _lib.ERR_INVALID_ARGUMENT
    assert g(a[0], a[1], a[0] + 512, a[3], None) == _lib.ERR_INVALID_ARGUMENT   # codes over W_gate
    assert g(a[0], a[1], a[2], a[2] + 256, None) == _lib.ERR_INVALID_ARGUMENT   # scales over codes
    assert d(a[0], a[1], a[1] + 4, None) == _lib.ERR_INVALID_ARGUMENT
    assert d(a[0], a[0] + 64, a[2], None) == _lib.ERR_INVALID_ARGUMENT


def test_experts_argument_checks(lib):
    # X, idx, w, W_gateup, W_down, out
    a = [_addr(i) for i in range(6)]
    N = 100
    need = lib.lfm_moe_workspace_bytes(N)
    ws = _addr(7)
    f = lib.lfm_moe_experts_ws
    assert f(*a, 0, None, 0, None) == _lib.OK                              # N == 0: nothing launched
    assert f(*a, -1, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert f(*a, (1 << 24) + 1, ws, 1 << 50, None) == _lib.ERR_INVALID_ARGUMENT
    for i in range(6):
        b = list(a)
        b[i] = None
        assert f(*b, N, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
        assert b"null" in lib.lfm_moe_last_error()
        b = list(a)
        b[i] = a[i] + 4
        assert f(*b, N, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
        assert b"aligned" in lib.lfm_moe_last_error()
    assert f(*a, N, ws, need - 1, None) == _lib.ERR_WORKSPACE_TOO_SMALL
    assert f(*a, N, None, need, None) == _lib.ERR_INVALID_ARGUMENT
    b = list(a)
    b[5] = a[1] + 256                                                      # out over the selections
    assert f(*b, N, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert b"routing" in lib.lfm_moe_last_error()
    for i in (0, 3, 4):                                                    # X, W_gateup, W_down
        assert f(*a, N, a[i] - 256, need, None) == _lib.ERR_INVALID_ARGUMENT
        assert b"workspace overlaps an input" in lib.lfm_moe_last_error()
    b = list(a)
    b[2] = ws + 1024                                                       # weights inside the workspace
    assert f(*b, N, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert b"workspace overlaps the routing" in lib.lfm_moe_last_error()
    # FP8: X, idx, w, codes_gu, scales_gu, codes_d, scales_d, out
    a8 = [_addr(i) for i in range(8)]
    g = lib.lfm_moe_experts_fp8_ws
    assert g(*a8, 0, None, 0, None) == _lib.OK
    for i in range(8):
        b = list(a8)
        b[i] = None
        assert g(*b, N, ws, need, None) == _lib.ERR_INVALID_ARGUMENT
    assert g(*a8, N, ws, need - 1, None) == _lib.ERR_WORKSPACE_TOO_SMALL
    b = list(a8)
    b[1] = ws                                                              # selections are the workspace
    assert g(*b, N, ws, need, None) == _lib.ERR_INVALID_ARGUMENT


def test_routing_replacement_rule():
    """The rule include/lfm_moe.h states for given selections, on its host
    mirror: ids modulo 64, repeats replaced by the lowest id not among the
    token's other ids, valid rows unchanged."""
    from parity import sanitize_routing
    got = sanitize_routing(np.array([[5, 5, 5, 5], [-1, 63, 3, 3], [0, 64, 128, 1],
                                     [7, 9, 11, 13], [2, 2, 0, 1]], dtype=np.int32))
    np.testing.assert_array_equal(got, [[5, 0, 1, 2], [63, 0, 3, 1], [0, 2, 3, 1],
                                        [7, 9, 11, 13], [2, 3, 0, 1]])
    rng = np.random.default_rng(0)
    raw = rng.integers(-300, 300, size=(5000, 4)).astype(np.int32)
    out = sanitize_routing(raw)
    assert np.all((out >= 0) & (out < 64))
    assert all(len(set(r)) == 4 for r in out.tolist())
    valid = np.array([rng.choice(64, 4, replace=False) for _ in range(500)], dtype=np.int32)
    np.testing.assert_array_equal(sanitize_routing(valid), valid)


def test_timing_read_checks_its_arguments(lib):
    assert lib.lfm_moe_timing_read(None, None) == _lib.ERR_INVALID_ARGUMENT


def test_release_without_allocation_is_a_no_op(lib):
    lib.lfm_moe_release()
