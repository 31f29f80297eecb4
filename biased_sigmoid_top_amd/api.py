"""Python face of the C ABI: same names as include/lfm_moe.h, torch tensors in.

PyTorch only provides device memory and streams here; every call goes
straight to the HIP library through ctypes.
"""

from __future__ import annotations

import torch

from . import _lib

HIDDEN, EXPERTS, TOP_K, FF = 2048, 64, 4, 1536


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _req(t: torch.Tensor, name: str, dtype, shape) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _weights(W_r, bias, W_gateup, W_down):
    return (_req(W_r, "W_r", torch.bfloat16, (EXPERTS, HIDDEN)),
            _req(bias, "bias", torch.float32, (EXPERTS,)),
            _req(W_gateup, "W_gateup (packed)", torch.bfloat16, (EXPERTS * 2 * FF * HIDDEN,)),
            _req(W_down, "W_down (packed)", torch.bfloat16, (EXPERTS * HIDDEN * FF,)))


def pack_gateup(W_gate, W_up, out=None, stream=None):
    """Packs [64, 1536, 2048] gate and up matrices into the fragment layout."""
    pg = _req(W_gate, "W_gate", torch.bfloat16, (EXPERTS, FF, HIDDEN))
    pu = _req(W_up, "W_up", torch.bfloat16, (EXPERTS, FF, HIDDEN))
    if out is None:
        out = torch.empty(EXPERTS * 2 * FF * HIDDEN, dtype=torch.bfloat16, device=W_gate.device)
    po = _req(out, "W_gateup", torch.bfloat16, (EXPERTS * 2 * FF * HIDDEN,))
    _lib.call("lfm_moe_pack_gateup", pg, pu, po, _stream(stream))
    return out


def pack_gateup_stacked(W_gateup, out=None, stream=None):
    """Packs one stacked [64, 3072, 2048] gate/up tensor (rows 0..1535 of an
    expert are its gate rows, 1536..3071 its up rows) into the fragment
    layout; the same bytes as pack_gateup on the two halves."""
    pw = _req(W_gateup, "W_gateup", torch.bfloat16, (EXPERTS, 2 * FF, HIDDEN))
    if out is None:
        out = torch.empty(EXPERTS * 2 * FF * HIDDEN, dtype=torch.bfloat16, device=W_gateup.device)
    po = _req(out, "W_gateup_packed", torch.bfloat16, (EXPERTS * 2 * FF * HIDDEN,))
    _lib.call("lfm_moe_pack_gateup_stacked", pw, po, _stream(stream))
    return out


def pack_down(W_down, out=None, stream=None):
    """Packs the [64, 2048, 1536] down matrices into the fragment layout."""
    pd = _req(W_down, "W_down", torch.bfloat16, (EXPERTS, HIDDEN, FF))
    if out is None:
        out = torch.empty(EXPERTS * HIDDEN * FF, dtype=torch.bfloat16, device=W_down.device)
    po = _req(out, "W_down_packed", torch.bfloat16, (EXPERTS * HIDDEN * FF,))
    _lib.call("lfm_moe_pack_down", pd, po, _stream(stream))
    return out


def abi_version() -> int:
    return _lib.load().lfm_moe_abi_version()


def workspace_bytes(N: int) -> int:
    return int(_lib.load().lfm_moe_workspace_bytes(N))


def workspace_offset(N: int, region: int) -> int:
    return int(_lib.load().lfm_moe_workspace_offset(N, region))


def alloc_workspace(N: int, device=None) -> torch.Tensor:
    """A byte tensor big enough for lfm_moe_forward_ws at N tokens."""
    return torch.empty(max(workspace_bytes(N), 256), dtype=torch.uint8,
                       device=device if device is not None else "cuda")


def workspace_view(ws: torch.Tensor, N: int, region: int, dtype, shape) -> torch.Tensor:
    """A typed view of one workspace region (see lfm_moe_ws_region)."""
    off = workspace_offset(N, region)
    n = 1
    for s in shape:
        n *= s
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype).view(*shape)


def rmsnorm(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    N = x.shape[0]
    px = _req(x, "x", torch.float32, (N, HIDDEN))
    if out is None:
        out = torch.empty(N, HIDDEN, dtype=torch.bfloat16, device=x.device)
    po = _req(out, "out", torch.bfloat16, (N, HIDDEN))
    _lib.call("lfm_moe_rmsnorm", px, po, N, _stream(stream))
    return out


def route_workspace_bytes(N: int) -> int:
    return int(_lib.load().lfm_moe_route_workspace_bytes(N))


def route(X, W_r, bias, idx=None, w=None, workspace=None, stream=None):
    """Selections [N, 4] int32 and weights [N, 4] fp32.  With ``workspace``
    (a byte tensor of at least route_workspace_bytes(N)) lfm_moe_route_ws is
    used."""
    N = X.shape[0]
    pX = _req(X, "X", torch.bfloat16, (N, HIDDEN))
    pW = _req(W_r, "W_r", torch.bfloat16, (EXPERTS, HIDDEN))
    pb = _req(bias, "bias", torch.float32, (EXPERTS,))
    if idx is None:
        idx = torch.empty(N, TOP_K, dtype=torch.int32, device=X.device)
    if w is None:
        w = torch.empty(N, TOP_K, dtype=torch.float32, device=X.device)
    pi = _req(idx, "idx", torch.int32, (N, TOP_K))
    pw = _req(w, "w", torch.float32, (N, TOP_K))
    if workspace is None:
        _lib.call("lfm_moe_route", pX, pW, pb, pi, pw, N, _stream(stream))
    else:
        _lib.call("lfm_moe_route_ws", pX, pW, pb, pi, pw, N, workspace.data_ptr(),
                  workspace.numel() * workspace.element_size(), _stream(stream))
    return idx, w


FP8_GATEUP_SCALES = (EXPERTS, 2, FF // 128, HIDDEN // 128)
FP8_DOWN_SCALES = (EXPERTS, HIDDEN // 128, FF // 128)


def pack_fp8_gateup(W_gate, W_up, stream=None):
    """FP8 block quantisation of the gate and up matrices: (codes [64*3072*2048]
    uint8 in the FP8 fragment layout, scales [64, 2, 12, 16] fp32)."""
    pg = _req(W_gate, "W_gate", torch.bfloat16, (EXPERTS, FF, HIDDEN))
    pu = _req(W_up, "W_up", torch.bfloat16, (EXPERTS, FF, HIDDEN))
    codes = torch.empty(EXPERTS * 2 * FF * HIDDEN, dtype=torch.uint8, device=W_gate.device)
    scales = torch.empty(FP8_GATEUP_SCALES, dtype=torch.float32, device=W_gate.device)
    _lib.call("lfm_moe_pack_fp8_gateup", pg, pu, codes.data_ptr(), scales.data_ptr(), _stream(stream))
    return codes, scales


def pack_fp8_gateup_stacked(W_gateup, stream=None):
    """FP8 block quantisation of one stacked [64, 3072, 2048] gate/up tensor:
    the same (codes, scales) as pack_fp8_gateup on its two halves."""
    pw = _req(W_gateup, "W_gateup", torch.bfloat16, (EXPERTS, 2 * FF, HIDDEN))
    codes = torch.empty(EXPERTS * 2 * FF * HIDDEN, dtype=torch.uint8, device=W_gateup.device)
    scales = torch.empty(FP8_GATEUP_SCALES, dtype=torch.float32, device=W_gateup.device)
    _lib.call("lfm_moe_pack_fp8_gateup_stacked", pw, codes.data_ptr(), scales.data_ptr(), _stream(stream))
    return codes, scales


def pack_fp8_down(W_down, stream=None):
    """FP8 block quantisation of the down matrices: (codes [64*2048*1536] uint8,
    scales [64, 16, 12] fp32)."""
    pd = _req(W_down, "W_down", torch.bfloat16, (EXPERTS, HIDDEN, FF))
    codes = torch.empty(EXPERTS * HIDDEN * FF, dtype=torch.uint8, device=W_down.device)
    scales = torch.empty(FP8_DOWN_SCALES, dtype=torch.float32, device=W_down.device)
    _lib.call("lfm_moe_pack_fp8_down", pd, codes.data_ptr(), scales.data_ptr(), _stream(stream))
    return codes, scales


def forward_fp8(X, W_r, bias, gateup_fp8, down_fp8, out=None, workspace=None, stream=None):
    """The layer with FP8 experts (any N up to FP8_MAX_TOKENS): gateup_fp8 and
    down_fp8 are the (codes, scales) pairs of pack_fp8_gateup /
    pack_fp8_down.  With ``workspace`` the _ws entry point is used."""
    N = X.shape[0]
    pX = _req(X, "X", torch.bfloat16, (N, HIDDEN))
    pr = _req(W_r, "W_r", torch.bfloat16, (EXPERTS, HIDDEN))
    pb = _req(bias, "bias", torch.float32, (EXPERTS,))
    gc = _req(gateup_fp8[0], "W_gateup_fp8", torch.uint8, (EXPERTS * 2 * FF * HIDDEN,))
    gs = _req(gateup_fp8[1], "scales_gateup", torch.float32, FP8_GATEUP_SCALES)
    dc = _req(down_fp8[0], "W_down_fp8", torch.uint8, (EXPERTS * HIDDEN * FF,))
    ds = _req(down_fp8[1], "scales_down", torch.float32, FP8_DOWN_SCALES)
    if out is None:
        out = torch.empty(N, HIDDEN, dtype=torch.float32, device=X.device)
    po = _req(out, "out", torch.float32, (N, HIDDEN))
    if workspace is None:
        _lib.call("lfm_moe_forward_fp8", pX, pr, pb, gc, gs, dc, ds, po, N, _stream(stream))
    else:
        _lib.call("lfm_moe_forward_fp8_ws", pX, pr, pb, gc, gs, dc, ds, po, N, workspace.data_ptr(),
                  workspace.numel() * workspace.element_size(), _stream(stream))
    return out


def _temporaries(out, workspace, N, device, stream):
    """The output and workspace of an expert-path call, allocated here when
    not given.  The caching allocator hands out memory for the current
    stream; when the call runs on another stream, the tensors are marked as
    in use there, so that their memory is not reused before that stream has
    passed the call."""
    made = []
    if out is None:
        out = torch.empty(N, HIDDEN, dtype=torch.float32, device=device)
        made.append(out)
    if workspace is None:
        workspace = alloc_workspace(N, device)
        made.append(workspace)
    if stream is not None:
        for t in made:
            t.record_stream(stream)
    return out, workspace


def _routing(idx, w, N):
    return (_req(idx, "idx", torch.int32, (N, TOP_K)), _req(w, "w", torch.float32, (N, TOP_K)))


def experts(X, idx, w, W_gateup, W_down, out=None, workspace=None, stream=None):
    """The expert path on caller-given routing (lfm_moe_experts_ws): idx
    [N, 4] int32, w [N, 4] fp32.  Without ``workspace`` one is allocated."""
    N = X.shape[0]
    pX = _req(X, "X", torch.bfloat16, (N, HIDDEN))
    pi, pw = _routing(idx, w, N)
    pg = _req(W_gateup, "W_gateup (packed)", torch.bfloat16, (EXPERTS * 2 * FF * HIDDEN,))
    pd = _req(W_down, "W_down (packed)", torch.bfloat16, (EXPERTS * HIDDEN * FF,))
    out, workspace = _temporaries(out, workspace, N, X.device, stream)
    po = _req(out, "out", torch.float32, (N, HIDDEN))
    _lib.call("lfm_moe_experts_ws", pX, pi, pw, pg, pd, po, N, workspace.data_ptr(),
              workspace.numel() * workspace.element_size(), _stream(stream))
    return out


def experts_fp8(X, idx, w, gateup_fp8, down_fp8, out=None, workspace=None, stream=None):
    """The FP8 expert path on caller-given routing (lfm_moe_experts_fp8_ws)."""
    N = X.shape[0]
    pX = _req(X, "X", torch.bfloat16, (N, HIDDEN))
    pi, pw = _routing(idx, w, N)
    gc = _req(gateup_fp8[0], "W_gateup_fp8", torch.uint8, (EXPERTS * 2 * FF * HIDDEN,))
    gs = _req(gateup_fp8[1], "scales_gateup", torch.float32, FP8_GATEUP_SCALES)
    dc = _req(down_fp8[0], "W_down_fp8", torch.uint8, (EXPERTS * HIDDEN * FF,))
    ds = _req(down_fp8[1], "scales_down", torch.float32, FP8_DOWN_SCALES)
    out, workspace = _temporaries(out, workspace, N, X.device, stream)
    po = _req(out, "out", torch.float32, (N, HIDDEN))
    _lib.call("lfm_moe_experts_fp8_ws", pX, pi, pw, gc, gs, dc, ds, po, N, workspace.data_ptr(),
              workspace.numel() * workspace.element_size(), _stream(stream))
    return out


def forward(X, W_r, bias, W_gateup, W_down, out=None, workspace=None, stream=None):
    """out [N, 2048] fp32.  With ``workspace`` the _ws entry point is used."""
    N = X.shape[0]
    pX = _req(X, "X", torch.bfloat16, (N, HIDDEN))
    pw = _weights(W_r, bias, W_gateup, W_down)
    if out is None:
        out = torch.empty(N, HIDDEN, dtype=torch.float32, device=X.device)
    po = _req(out, "out", torch.float32, (N, HIDDEN))
    if workspace is None:
        _lib.call("lfm_moe_forward", pX, *pw, po, N, _stream(stream))
    else:
        _lib.call("lfm_moe_forward_ws", pX, *pw, po, N, workspace.data_ptr(),
                  workspace.numel() * workspace.element_size(), _stream(stream))
    return out


def block_forward(x, W_r, bias, W_gateup, W_down, workspace=None, stream=None):
    """x <- x + MoE(bf16(RMSNorm(x))) in place; returns x."""
    N = x.shape[0]
    px = _req(x, "x", torch.float32, (N, HIDDEN))
    pw = _weights(W_r, bias, W_gateup, W_down)
    if workspace is None:
        _lib.call("lfm_moe_block_forward", px, *pw, N, _stream(stream))
    else:
        _lib.call("lfm_moe_block_forward_ws", px, *pw, N, workspace.data_ptr(),
                  workspace.numel() * workspace.element_size(), _stream(stream))
    return x


def _ws_args(workspace):
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def stage_dispatch(idx, w, workspace, stream=None):
    """Routing copy + dispatch into the workspace regions (lfm_moe_stage_dispatch)."""
    N = idx.shape[0]
    pi = _req(idx, "idx", torch.int32, (N, TOP_K))
    pw = _req(w, "w", torch.float32, (N, TOP_K))
    _lib.call("lfm_moe_stage_dispatch", pi, pw, N, *_ws_args(workspace), _stream(stream))


def stage_gateup(X, W_gateup, workspace, stream=None):
    """X and the workspace's grouping -> H region (lfm_moe_stage_gateup)."""
    N = X.shape[0]
    pX = _req(X, "X", torch.bfloat16, (N, HIDDEN))
    pg = _req(W_gateup, "W_gateup (packed)", torch.bfloat16, (EXPERTS * 2 * FF * HIDDEN,))
    _lib.call("lfm_moe_stage_gateup", pX, pg, N, *_ws_args(workspace), _stream(stream))


def stage_down(W_down, N, workspace, stream=None):
    """H region -> Y region (lfm_moe_stage_down)."""
    pd = _req(W_down, "W_down (packed)", torch.bfloat16, (EXPERTS * HIDDEN * FF,))
    _lib.call("lfm_moe_stage_down", pd, N, *_ws_args(workspace), _stream(stream))


def stage_combine(N, workspace, out=None, resid=None, stream=None):
    """Y and W regions -> out [N, 2048] fp32 (lfm_moe_stage_combine)."""
    if out is None:
        out = torch.empty(N, HIDDEN, dtype=torch.float32, device=workspace.device)
    po = _req(out, "out", torch.float32, (N, HIDDEN))
    pr = _req(resid, "resid", torch.float32, (N, HIDDEN)) if resid is not None else None
    _lib.call("lfm_moe_stage_combine", pr, po, N, *_ws_args(workspace), _stream(stream))
    return out


def stack_forward(x, blocks, workspace=None, stream=None):
    """x <- x + MoE_l(bf16(RMSNorm(x))) for each (W_r, bias, W_gateup, W_down)
    of ``blocks`` in order, in place; returns x.  Without ``workspace`` one of
    workspace_bytes(N) is allocated for the call."""
    import ctypes
    N = x.shape[0]
    px = _req(x, "x", torch.float32, (N, HIDDEN))
    arr = (_lib.BlockWeights * max(1, len(blocks)))()
    for i, blk in enumerate(blocks):
        arr[i] = _lib.BlockWeights(*_weights(*blk))
    if workspace is None:
        workspace = alloc_workspace(N, device=x.device)
    _lib.call("lfm_moe_stack_forward_ws", px, ctypes.addressof(arr), len(blocks), N, workspace.data_ptr(),
              workspace.numel() * workspace.element_size(), _stream(stream))
    return x


def release() -> None:
    _lib.load().lfm_moe_release()


def timing_enable(on: bool) -> None:
    """Per-kernel event timing of later layer calls (clears the totals)."""
    _lib.call("lfm_moe_timing_enable", 1 if on else 0)


def timing_read() -> dict:
    """{stage: (total_ms, launches)} of the calls timed since timing_enable."""
    import ctypes
    ms = (ctypes.c_double * len(_lib.STAGES))()
    n = (ctypes.c_int64 * len(_lib.STAGES))()
    _lib.call("lfm_moe_timing_read", ctypes.addressof(ms), ctypes.addressof(n))
    return {s: (ms[i], n[i]) for i, s in enumerate(_lib.STAGES)}
