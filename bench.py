#!/usr/bin/env python3
"""Throughput of the biased-sigmoid top-4 MoE layer on one MI355X.

One step = one lfm_moe_forward (router, dispatch, gate/up, down, combine)
over one batch of synthetic tokens whose inputs and weights are already
resident in HBM.  The headline workload is the decode-shaped layer (N = 64
tokens, seed 1); the prefill-shaped layer (N = 4096, seed 2) and the same
decode layer with FP8 block-scaled experts are measured in the same run and
reported beside it.  Expert weights are cycled over
`--copies` identical device copies so that the 256 MB Infinity Cache does
not serve repeated steps.

Prints ONE JSON line (rank 0, N = 1 GPU).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at N=64 and N=4096; % HBM BW / % bf16 MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (the FP8 layer's grouped kernels)

D, E, K, FF = 2048, 64, 4, 1536
GATEUP_W_BYTES = 2 * FF * D * 2            # 12,582,912 per active expert
DOWN_W_BYTES = D * FF * 2                  # 6,291,456 per active expert
EXPERT_BYTES = GATEUP_W_BYTES + DOWN_W_BYTES  # 18,874,368
ROUTER_BYTES = E * D * 2 + E * 4
FLOP_PER_TOKEN = 2 * E * D + K * 2 * 3 * D * FF  # 75,759,616


def layer_bytes(A, N):
    """Algorithmic HBM bytes of one layer call: active experts' weights once,
    the router, x read in bf16 and out written in fp32."""
    return A * EXPERT_BYTES + ROUTER_BYTES + N * (D * 2 + D * 4)


def gateup_bytes(A, N):
    """Algorithmic bytes of the gate/up kernel: active gate/up weights once,
    the token rows once, H written once in bf16."""
    return A * GATEUP_W_BYTES + N * D * 2 + K * N * FF * 2


def gateup_flops(N):
    return K * N * 2 * (2 * FF) * D


# FP8 experts: one byte per weight plus a fp32 scale per 128 x 128 block.
FP8_GATEUP_W_BYTES = 2 * FF * D + 2 * (FF // 128) * (D // 128) * 4   # 6,292,992 per active expert
FP8_DOWN_W_BYTES = D * FF + (D // 128) * (FF // 128) * 4             # 3,146,496 per active expert


def fp8_layer_bytes(A, N):
    return A * (FP8_GATEUP_W_BYTES + FP8_DOWN_W_BYTES) + ROUTER_BYTES + N * (D * 2 + D * 4)


FP8_STREAM = 4  # FP8 layer: weight-streaming kernels up to this many tokens


def fp8_act_bytes(rows, width, N):
    """Bytes of the rows an FP8 kernel reads: bf16 for the weight-streaming
    kernels (they quantise in registers), E4M3 codes plus a fp32 scale per
    128 values for the grouped ones."""
    return rows * width * 2 if N <= FP8_STREAM else rows * (width + width // 128 * 4)


def fp8_gateup_bytes(A, N):
    return A * FP8_GATEUP_W_BYTES + fp8_act_bytes(N, D, N) + K * N * FF * 2


def fp8_down_bytes(A, N):
    return A * FP8_DOWN_W_BYTES + fp8_act_bytes(K * N, FF, N) + K * N * D * 4


def down_bytes(A, N):
    return A * DOWN_W_BYTES + K * N * FF * 2 + K * N * D * 4


def down_flops(N):
    return K * N * 2 * D * FF


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prepare(name, copies, zero_bias=False):
    import torch
    import synth
    w = synth.WORKLOADS[name]
    N = w["N"]
    log(f"generating {name}: N={N} seed={w['seed']} skew={w['skew']}"
        + (" with the bias set to zero" if zero_bias else ""))
    layer = synth.layer_inputs(N, w["seed"], w["skew"])
    if zero_bias:
        layer["bias"] = torch.zeros_like(layer["bias"])
    return prepare_layer(name, N, w["seed"], layer, copies)


def expert_counts(p, N):
    """Slots per expert of the first N tokens (one untimed call through the _ws form)."""
    import torch
    import biased_sigmoid_top_amd as moe
    from biased_sigmoid_top_amd import _lib
    ws = moe.alloc_workspace(N)
    moe.forward(p["X"][:N], p["W_r"], p["bias"], p["Wgu"][0], p["Wd"][0], p["out"][:N], workspace=ws)
    sel = moe.workspace_view(ws, N, _lib.WS_IDX, torch.int32, (N, 4)).cpu().long()
    del ws
    torch.cuda.synchronize()
    return torch.bincount(sel.reshape(-1), minlength=E).tolist()


def inputs_sha256(layer):
    """SHA-256 over the generated tensors of a workload (z, W_r, bias, W_gate,
    W_up, W_down, in that order): the same digest on two machines means the
    same inputs."""
    import hashlib
    import torch
    h = hashlib.sha256()
    for k in ("z", "W_r", "bias", "W_gate", "W_up", "W_down"):
        h.update(layer[k].contiguous().view(-1).view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


def prepare_layer(name, N, seed, layer, copies):
    import torch
    import biased_sigmoid_top_amd as moe
    dev = torch.device("cuda")
    X = moe.rmsnorm(layer["z"].to(dev))          # input preparation, not timed
    W_r, bias = layer["W_r"].to(dev), layer["bias"].to(dev)
    Wgu0 = moe.pack_gateup(layer["W_gate"].to(dev), layer["W_up"].to(dev))
    Wd0 = moe.pack_down(layer["W_down"].contiguous().to(dev))
    Wgu = [Wgu0] + [Wgu0.clone() for _ in range(copies - 1)]
    Wd = [Wd0] + [Wd0.clone() for _ in range(copies - 1)]
    out = torch.empty(N, D, dtype=torch.float32, device=dev)
    p = dict(name=name, N=N, seed=seed, layer=layer, X=X, W_r=W_r, bias=bias,
             Wgu=Wgu, Wd=Wd, out=out)
    p["counts"] = expert_counts(p, N)
    return p


def prepare_fp8(p):
    """FP8 codes and scales of a prepared workload's experts (packed on the
    device), one set per weight copy."""
    import biased_sigmoid_top_amd as moe
    import torch
    layer = p["layer"]
    dev = torch.device("cuda")
    gu = moe.pack_fp8_gateup(layer["W_gate"].to(dev), layer["W_up"].to(dev))
    dn = moe.pack_fp8_down(layer["W_down"].contiguous().to(dev))
    c = len(p["Wgu"])
    q = dict(p, fp8=True,
             Gq=[gu] + [tuple(t.clone() for t in gu) for _ in range(c - 1)],
             Dq=[dn] + [tuple(t.clone() for t in dn) for _ in range(c - 1)])
    return q


def time_steps(p, steps, warmup, min_warm_ms=0.0):
    """warmup untimed steps (continued, for a large workload, until they have
    taken min_warm_ms), then the timed steps."""
    import torch
    import biased_sigmoid_top_amd as moe
    c = len(p["Wgu"])

    def step(i):
        if p.get("fp8"):
            moe.forward_fp8(p["X"], p["W_r"], p["bias"], p["Gq"][i % c], p["Dq"][i % c], p["out"])
        else:
            moe.forward(p["X"], p["W_r"], p["bias"], p["Wgu"][i % c], p["Wd"][i % c], p["out"])

    tw = time.perf_counter()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    i = warmup
    while (time.perf_counter() - tw) * 1e3 < min_warm_ms:
        step(i)
        i += 1
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps

    # Second pass over the same steps with per-kernel hipEvents recorded by
    # the library on the launch stream.
    moe.timing_enable(True)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    stages = moe.timing_read()
    moe.timing_enable(False)
    per_kernel = {s: (ms / n if n else 0.0) for s, (ms, n) in stages.items()}
    assert torch.isfinite(p["out"]).all().item(), "non-finite layer output"

    # Third pass: per-step device times from event pairs around each step.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        step(i)
        b.record()
    torch.cuda.synchronize()
    per_kernel["step_percentiles_ms"] = percentiles([a.elapsed_time(b) for a, b in evs])
    return wall_ms, per_kernel


def percentiles(xs):
    """p10 / median / p90 of per-step times (ms)."""
    import numpy as np
    q = np.percentile(np.asarray(xs, dtype=np.float64), [10, 50, 90])
    return dict(p10=float(q[0]), p50=float(q[1]), p90=float(q[2]))


def summarize(p, wall_ms, per_kernel):
    N = p["N"]
    A = sum(1 for c in p["counts"] if c > 0)
    s = wall_ms * 1e-3
    tok_s = N / s
    gbs = layer_bytes(A, N) / s / 1e9
    tflops = N * FLOP_PER_TOKEN / s / 1e12
    gu_ms = per_kernel["gateup"]
    dn_ms = per_kernel["down"]
    return dict(
        N=N, active_experts=A, max_tokens_per_expert=max(p["counts"]),
        ms_per_step=wall_ms, tokens_per_s=tok_s,
        layer_gbs=gbs, layer_hbm_frac=gbs / HBM_PEAK_GBS,
        layer_tflops=tflops, layer_mfma_frac=tflops / BF16_PEAK_TFLOPS,
        kernel_ms=per_kernel,
        gateup_gbs=gateup_bytes(A, N) / (gu_ms * 1e-3) / 1e9 if gu_ms else None,
        gateup_tflops=gateup_flops(N) / (gu_ms * 1e-3) / 1e12 if gu_ms else None,
        down_gbs=down_bytes(A, N) / (dn_ms * 1e-3) / 1e9 if dn_ms else None,
        down_tflops=down_flops(N) / (dn_ms * 1e-3) / 1e12 if dn_ms else None,
    )




def summarize_fp8(p, wall_ms, per_kernel, label, note):
    """Summary of FP8-expert steps: bytes are the FP8 codes and scales of the
    active experts, the router, x in and out; FLOPs are the layer's.  The
    weight-streaming kernels (HBM-bound) widen the codes to bf16; the grouped
    kernels (MFMA-bound) run on the FP8 matrix core, whose dense peak they
    are measured against."""
    N = p["N"]
    A = sum(1 for c in p["counts"] if c > 0)
    s = wall_ms * 1e-3
    gu_ms, dn_ms = per_kernel["gateup"], per_kernel["down"]
    gu_gbs = fp8_gateup_bytes(A, N) / (gu_ms * 1e-3) / 1e9
    gu_tflops = gateup_flops(N) / (gu_ms * 1e-3) / 1e12
    gbs = fp8_layer_bytes(A, N) / s / 1e9
    tflops = N * FLOP_PER_TOKEN / s / 1e12
    hbm = tflops * 1e3 / gbs < 0.5 * FP8_PEAK_TFLOPS * 1e3 / HBM_PEAK_GBS
    kernel = "gateup_decode_fp8" if N <= FP8_STREAM else "gateup_tiled_fp8"
    if hbm:
        roof = dict(bound="hbm", kernel=kernel, achieved=gu_gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=gu_gbs / HBM_PEAK_GBS,
                    traffic=measured_traffic(p["name"], "gateup_fp8", KERNEL_SOURCE[kernel]),
                    bytes_per_launch=fp8_gateup_bytes(A, N), avg_launch_ms=gu_ms, timing=EVENT_TIMING,
                    down_gbs=fp8_down_bytes(A, N) / (dn_ms * 1e-3) / 1e9)
    else:
        roof = dict(bound="mfma", kernel=kernel, achieved=gu_tflops, peak=FP8_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=gu_tflops / FP8_PEAK_TFLOPS, traffic=None,
                    flops_per_launch=gateup_flops(N), avg_launch_ms=gu_ms, timing=EVENT_TIMING)
    return dict(config=label, N=N, dtype="fp8-e4m3 experts (bf16 router)",
                active_experts=A, max_tokens_per_expert=max(p["counts"]), ms_per_step=wall_ms,
                tokens_per_s=N / s, gbs=gbs, hbm_frac=gbs / HBM_PEAK_GBS, tflops=tflops,
                mfma_frac=tflops / FP8_PEAK_TFLOPS, bound="hbm" if hbm else "mfma",
                roofline_frac=gbs / HBM_PEAK_GBS if hbm else tflops / FP8_PEAK_TFLOPS,
                kernel_ms=per_kernel, roofline=roof, note=note)


def measure_fp8(p, steps, warmup, label, note, q=None, min_warm_ms=0.0):
    """FP8 steps on workload p (packing its experts unless q, a prepare_fp8
    result of the same layer, is given)."""
    q = prepare_fp8(p) if q is None else dict(q, N=p["N"], X=p["X"], out=p["out"], counts=p["counts"])
    log(f"timing {label} (FP8 experts, {p['name']}): {steps} steps")
    w, k = time_steps(q, steps, warmup, min_warm_ms)
    e = summarize_fp8(q, w, k, label, note)
    log(json.dumps(e))
    del q
    return e


# Source file of each dominant kernel named in the roofline objects.
KERNEL_SOURCE = {"gateup_decode": "expert_stream.hip", "gateup_tiled": "expert_tiled.hip",
                 "gateup_decode_fp8": "expert_stream.hip", "gateup_tiled_fp8": "expert_tiled.hip"}


def kernel_source_digest(path):
    import hashlib
    with open(os.path.join(ROOT, "biased_sigmoid_top_amd", "csrc", path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload, kernel, source):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter
    summary of this workload, or None when it is missing, was taken on
    another kernel (source file) or on a different version of its source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    start = text.find("```json")
    if start < 0:
        return None
    rec = json.loads(text[start + 7:text.index("```", start + 7)])
    if rec.get("source") != source or rec.get("source_digest") != kernel_source_digest(source):
        return None
    return rec["hbm_bytes_per_launch"]


def roofline(h, workload):
    """Roofline object of the dominant kernel (gate/up): HBM-bound while the
    arithmetic intensity is far below the ridge (hbm_bound), bf16-MFMA-bound
    otherwise."""
    from biased_sigmoid_top_amd._lib import DECODE_MAX_TOKENS
    N, A = h["N"], h["active_experts"]
    ms = h["kernel_ms"]["gateup"]
    if hbm_bound(h):
        kernel = "gateup_decode" if N <= DECODE_MAX_TOKENS else "gateup_tiled"
        return dict(bound="hbm", kernel=kernel, achieved=h["gateup_gbs"],
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=h["gateup_gbs"] / HBM_PEAK_GBS,
                    traffic=measured_traffic(workload, "gateup", KERNEL_SOURCE[kernel]),
                    bytes_per_launch=gateup_bytes(A, N),
                    avg_launch_ms=ms, timing=EVENT_TIMING)
    return dict(bound="mfma", kernel="gateup_tiled", achieved=h["gateup_tflops"],
                peak=BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=h["gateup_tflops"] / BF16_PEAK_TFLOPS,
                traffic=measured_traffic(workload, "gateup", KERNEL_SOURCE["gateup_tiled"]),
                flops_per_launch=gateup_flops(N),
                avg_launch_ms=ms, timing=EVENT_TIMING)


# How avg_launch_ms is measured (stated in every roofline object).
EVENT_TIMING = ("hipEvents recorded by the library on the launch stream before the layer's first "
                "kernel and after each kernel, over a second pass of the timed steps: a kernel's "
                "interval includes the dispatch gap before it (about 1-4 us), so it reads a little "
                "above the kernel-only duration in the rocprofv3 traces under profiles/")


def cpu_baseline(p, budget_s):
    """The oracle as it stands, timed on this host's cores on the same workload."""
    import numpy as np
    import threadpoolctl
    import oracle
    layer = p["layer"]
    X = oracle.block_input(layer["z"].numpy())
    args = (X, layer["W_r"].float().numpy(), layer["bias"].numpy(), layer["W_gate"].float().numpy(),
            layer["W_up"].float().numpy(), layer["W_down"].float().numpy())
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.moe_forward(*args)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()
                   if i.get("user_api") == "blas"), default=1)
    return dict(value=reps * p["N"] / el, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"{reps} whole-layer oracle forwards of the {p['name']} workload "
                       f"({p['N']} tokens each, float64 NumPy), {el:.1f} s")


def device_info():
    """The device as torch reports it, plus (best effort) the clocks and
    power that rocm-smi reports right after the timed work: boxes of the
    same model measured up to ~20% apart, and this records what differed."""
    import subprocess
    import torch
    p = torch.cuda.get_device_properties(0)
    info = dict(name=p.name, arch=getattr(p, "gcnArchName", None), cus=p.multi_processor_count,
                memory_gib=round(p.total_memory / 2**30, 1), smi=None)
    # Under rocprofv3 a child process inherits the profiler's preloaded
    # library, which opens the GPU before rocm-smi's interpreter starts; skip
    # the query there (the profile does not need it).
    if any(k.startswith("ROCPROF") for k in os.environ):
        return info
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--showtemp", "--json"],
                           capture_output=True, text=True, timeout=20)
        if r.returncode == 0:
            info["smi"] = json.loads(r.stdout)
    except (OSError, subprocess.SubprocessError, ValueError):
        pass
    return info


def copy_probe():
    """A plain 1 GiB device copy, for calibrating HBM byte counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 3}))


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=3, help="device copies of the expert weights")
    ap.add_argument("--secondary", default="prefill_n4096",
                    help="second workload reported beside the headline one ('none' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the oracle baseline (0 leaves it out)")
    ap.add_argument("--copy-probe", action="store_true", help="only run a plain 1 GiB copy")
    ap.add_argument("--no-extra", action="store_true",
                    help="leave out the skewed 16,384-token layer and the 38-block stack (measured by default)")
    ap.add_argument("--workload", default="decode_n64", help="headline workload")
    ap.add_argument("--stack-only", action="store_true",
                    help="only measure the 38-block stack (for profiling it on its own); prints its entry")
    ap.add_argument("--configs", action="store_true",
                    help="also measure every configuration (C0-C4, the 38-block stack included; "
                         "several minutes) and add them, with the verification-batch series V1-V64, to the line under 'configs'")
    return ap.parse_args(argv)


def main():
    args = parse_args()

    if args.gpus != 1:
        print("bench.py measures one MI355X; it does not run on several GPUs (the layer would "
              "shard by tokens, or by experts with an all-to-all, across them).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs the GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return

    import biased_sigmoid_top_amd  # noqa: F401  (fails loudly without the built library)

    if args.stack_only:
        print(json.dumps(measure_stack(max(3, args.steps // 4), 1)), flush=True)
        return

    head = prepare(args.workload, args.copies)
    log(f"timing {args.workload}: {args.steps} steps after {args.warmup} warm-up")
    wall_ms, per_kernel = time_steps(head, args.steps, args.warmup)
    h = summarize(head, wall_ms, per_kernel)
    dev_info = device_info()
    h["inputs_sha256"] = inputs_sha256(head["layer"])
    log(json.dumps(h))

    from biased_sigmoid_top_amd._lib import FP8_MAX_TOKENS
    fp8 = None
    if head["N"] <= FP8_MAX_TOKENS:
        fp8 = measure_fp8(head, args.steps, args.warmup, "F1",
                          f"supplementary: {args.workload} with FP8 block-scaled experts")

    second = None
    if args.secondary != "none":
        p2 = prepare(args.secondary, args.copies)
        steps2 = max(5, args.steps // 10)
        log(f"timing {args.secondary}: {steps2} steps")
        w2, k2 = time_steps(p2, steps2, long_warmup(args), LONG_WARM_MS)
        second = summarize(p2, w2, k2)
        log(json.dumps(second))
        del p2
        torch.cuda.empty_cache()

    cpu = None
    if args.cpu_seconds > 0:
        log(f"timing the oracle for ~{args.cpu_seconds:.0f} s on host cores")
        cpu = cpu_baseline(head, args.cpu_seconds)

    line = build_line(args, h, head["seed"], second, cpu)
    line["fp8"] = fp8
    line["device"] = dev_info
    del head
    torch.cuda.empty_cache()
    if not args.no_extra:
        p3 = prepare("skewed_n16384", args.copies)
        steps3 = max(5, args.steps // 10)
        log(f"timing skewed_n16384: {steps3} steps")
        w3, k3 = time_steps(p3, steps3, long_warmup(args), LONG_WARM_MS)
        s3 = summarize(p3, w3, k3)
        line["skewed"] = dict(config_entry("C3", s3), workload="skewed_n16384",
                              roofline=roofline(s3, "skewed_n16384"))
        log(json.dumps(line["skewed"]))
        del p3
        torch.cuda.empty_cache()
        line["stack"] = measure_stack(max(3, args.steps // 4), 1)
        log(json.dumps(line["stack"]))
    if args.configs:
        line["configs"] = measure_configs(args)
    print(json.dumps(line), flush=True)


def long_warmup(args):
    """Untimed steps before the few timed steps of a large workload: at least
    two passes over the weight copies, and at least LONG_WARM_MS of them, so
    that no copy is first used, and the clock is not still rising, inside
    the timed region."""
    return max(2 * args.copies, args.warmup // 10)


LONG_WARM_MS = 30.0


def build_line(args, h, seed, second=None, cpu=None):
    """The one JSON result line from the measured summaries."""
    line = dict(
        metric=METRIC, value=h["tokens_per_s"], unit="tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=h["ms_per_step"], higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload=args.workload, N=h["N"], d=D, experts=E, top_k=K, ff=FF, seed=seed,
                    inputs_sha256=h.get("inputs_sha256"),
                    active_experts=h["active_experts"],
                    max_tokens_per_expert=h["max_tokens_per_expert"], weight_copies=args.copies),
        layer=dict(gbs=h["layer_gbs"], hbm_frac=h["layer_hbm_frac"], tflops=h["layer_tflops"],
                   mfma_frac=h["layer_mfma_frac"], kernel_ms=h["kernel_ms"]),
        roofline=roofline(h, args.workload), cpu_baseline=cpu,
    )
    if second is not None:
        line["prefill"] = dict(
            workload=args.secondary, N=second["N"], active_experts=second["active_experts"],
            ms_per_step=second["ms_per_step"], tokens_per_s=second["tokens_per_s"],
            gbs=second["layer_gbs"], hbm_frac=second["layer_hbm_frac"],
            tflops=second["layer_tflops"], mfma_frac=second["layer_mfma_frac"],
            kernel_ms=second["kernel_ms"],
            roofline=roofline(second, args.secondary))
    return line


# Every configuration of the layer contract: (label, workload, zero bias, note).
CONFIGS = (
    ("C0", "tiny_n32", False, None),
    ("C1", "decode_n64", False, None),
    ("C1u", "decode_n64", True, "supplementary: decode_n64 with the bias set to zero, so that "
                                "nearly all 64 experts are active"),
    ("C2", "prefill_n4096", False, None),
    ("C3", "skewed_n16384", False, None),
)


def hbm_bound(h):
    """HBM-bound while the layer's algorithmic intensity (FLOP per byte) is
    below half the ridge point of the two peaks (2.5 PFLOP/s / 8 TB/s = 312
    FLOP/B): decode and verification batches up to a few hundred tokens per
    expert; the N = 4096 and N = 16384 workloads sit at or above the ridge."""
    return h["layer_tflops"] * 1e3 / h["layer_gbs"] < 0.5 * BF16_PEAK_TFLOPS * 1e3 / HBM_PEAK_GBS


def config_entry(label, h, note=None):
    hbm = hbm_bound(h)
    e = dict(config=label, N=h["N"], active_experts=h["active_experts"],
             max_tokens_per_expert=h["max_tokens_per_expert"], ms_per_step=h["ms_per_step"],
             tokens_per_s=h["tokens_per_s"], gbs=h["layer_gbs"], hbm_frac=h["layer_hbm_frac"],
             tflops=h["layer_tflops"], mfma_frac=h["layer_mfma_frac"],
             bound="hbm" if hbm else "mfma",
             roofline_frac=h["layer_hbm_frac"] if hbm else h["layer_mfma_frac"],
             kernel_ms=h["kernel_ms"])
    if note:
        e["note"] = note
    return e


def measure_stack(steps, warmup):
    """The 38-block stack at N = 512: x <- x + MoE_l(bf16(RMSNorm(x))) for
    l = 0..37, each block with its own experts (about 46 GB resident)."""
    from concurrent.futures import ThreadPoolExecutor
    import torch
    import synth
    import biased_sigmoid_top_amd as moe
    from biased_sigmoid_top_amd import _lib
    st = synth.STACK
    N, nb = st["N"], st["blocks"]
    dev = torch.device("cuda")
    log(f"generating the stack: {nb} blocks at N={N} seed={st['seed']}")
    blocks = []
    with ThreadPoolExecutor(4) as pool:
        for bp in pool.map(lambda l: synth.stack_block_params(st["seed"], l), range(nb)):
            blocks.append((bp["W_r"].to(dev), bp["bias"].to(dev),
                           moe.pack_gateup(bp["W_gate"].to(dev), bp["W_up"].to(dev)),
                           moe.pack_down(bp["W_down"].contiguous().to(dev))))
            del bp
            if len(blocks) % 8 == 0:
                log(f"  {len(blocks)} blocks on the device")
    x0 = synth.stack_residual(N, st["seed"]).to(dev)
    x = x0.clone()
    ws = moe.alloc_workspace(N)
    active = []
    for blk in blocks:  # untimed pass: active experts of every block
        moe.block_forward(x, *blk, workspace=ws)
        sel = moe.workspace_view(ws, N, _lib.WS_IDX, torch.int32, (N, 4)).cpu().long()
        active.append(int((torch.bincount(sel.reshape(-1), minlength=E) > 0).sum()))
    del ws

    ws = moe.alloc_workspace(N)

    def stack_pass():
        x.copy_(x0)
        moe.stack_forward(x, blocks, workspace=ws)

    for _ in range(warmup):
        stack_pass()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        stack_pass()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    assert torch.isfinite(x).all().item(), "non-finite stack output"
    eager_x = x.clone()

    # The same stack captured once in a HIP graph (the library records no
    # allocation, memset or host synchronisation) and replayed.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        stack_pass()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stack_pass()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(x, eager_x), "graph replay differs from the eager stack"
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    ms_graph = (time.perf_counter() - t0) * 1e3 / steps
    assert torch.equal(x, eager_x), "graph replay differs from the eager stack"
    del graph
    # Per-kernel times of the blocks (library events), for the roofline of
    # the dominant kernel: gate/up, HBM-bound at 512 tokens.
    moe.timing_enable(True)
    stack_pass()
    torch.cuda.synchronize()
    st_ms = moe.timing_read()
    moe.timing_enable(False)
    kernel_ms = {k: (v / n if n else 0.0) for k, (v, n) in st_ms.items()}
    gu_bytes = sum(gateup_bytes(a, N) for a in active) / nb
    gu_ms = kernel_ms["gateup"]
    roof = dict(bound="hbm", kernel="gateup_tiled", achieved=gu_bytes / (gu_ms * 1e-3) / 1e9,
                peak=HBM_PEAK_GBS, unit="GB/s", frac=gu_bytes / (gu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                traffic=None, bytes_per_launch=gu_bytes, avg_launch_ms=gu_ms, timing=EVENT_TIMING)
    bytes_ = sum(a * EXPERT_BYTES + ROUTER_BYTES for a in active) + nb * N * D * 4 * 2
    flops = nb * N * FLOP_PER_TOKEN
    s = ms * 1e-3
    e = dict(config="C4", N=N, blocks=nb, active_experts_per_block_mean=sum(active) / nb,
             active_experts_per_block_min=min(active), active_experts_per_block_max=max(active),
             ms_per_step=ms, ms_per_block=ms / nb, tokens_per_s=N / s, gbs=bytes_ / s / 1e9,
             hbm_frac=bytes_ / s / 1e9 / HBM_PEAK_GBS, tflops=flops / s / 1e12,
             mfma_frac=flops / s / 1e12 / BF16_PEAK_TFLOPS, bound="hbm",
             roofline_frac=bytes_ / s / 1e9 / HBM_PEAK_GBS,
             ms_per_step_graph=ms_graph, tokens_per_s_graph=N / (ms_graph * 1e-3),
             kernel_ms=kernel_ms, roofline=roof,
             note="one step = the whole stack (a copy of x0, then one lfm_moe_stack_forward_ws call "
                  "over the 38 blocks: one normalisation launch, the later blocks' inputs normalised by "
                  "the previous block's combine); the _graph figures replay the same step captured in "
                  "one HIP graph")
    del blocks
    torch.cuda.empty_cache()
    return e


def measure_configs(args):
    import torch
    out = []
    for label, name, zero_bias, note in CONFIGS:
        p = prepare(name, args.copies, zero_bias)
        steps = args.steps if p["N"] <= 512 else max(5, args.steps // 10)
        log(f"timing {label} ({name}): {steps} steps")
        w, k = (time_steps(p, steps, args.warmup) if p["N"] <= 512 else
                time_steps(p, steps, long_warmup(args), LONG_WARM_MS))
        e = config_entry(label, summarize(p, w, k), note)
        log(json.dumps(e))
        out.append(e)
        if label == "C1u":
            out.append(measure_fp8(p, steps, args.warmup, "F1u",
                                   "supplementary: C1u with FP8 block-scaled experts"))
        if label == "C2":
            out.append(measure_fp8(p, steps, long_warmup(args), "F2",
                                   "supplementary: C2 with FP8 block-scaled experts (grouped kernels "
                                   "in FP8 mode)", min_warm_ms=LONG_WARM_MS))
        del p
        torch.cuda.empty_cache()
    e = measure_stack(max(3, args.steps // 40), 1)
    log(json.dumps(e))
    out.append(e)
    out += measure_verify(args)
    return out


def measure_verify(args):
    """Verification-shaped batches of speculative decoding: c requests x 10
    tokens per step, the first 10c tokens of one layer (seed 5)."""
    import torch
    import synth
    log("generating the verification-batch layer (seed 5)")
    Nmax = max(synth.verify_batch_sizes())
    from biased_sigmoid_top_amd._lib import FP8_MAX_TOKENS
    full = prepare_layer("verify", Nmax, synth.VERIFY["seed"], synth.verify_inputs(), args.copies)
    q = prepare_fp8(full)
    out = []
    for c, N in zip(synth.VERIFY["concurrency"], synth.verify_batch_sizes()):
        p = dict(full, N=N, X=full["X"][:N], out=full["out"][:N])
        p["counts"] = expert_counts(p, N)
        log(f"timing V{c}: {N} tokens, {args.steps} steps")
        w, k = time_steps(p, args.steps, args.warmup)
        e = config_entry(f"V{c}", summarize(p, w, k),
                         f"verification batch: {c} requests x 10 tokens (supplementary)")
        log(json.dumps(e))
        out.append(e)
        if N <= FP8_MAX_TOKENS:
            out.append(measure_fp8(p, args.steps, args.warmup, f"FV{c}",
                                   f"verification batch: {c} requests x 10 tokens, FP8 experts "
                                   "(supplementary)", q))
    del full, q
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
