"""bench.py host logic on the CPU: argument handling, algorithmic byte and
FLOP counts, roofline selection and the JSON line (no GPU)."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2
    assert "one MI355X" in r.stderr


def test_algorithmic_counts():
    # Per active expert: 3 x 2048 x 1536 bf16 weights (guide: 9,437,184 weights).
    assert bench.EXPERT_BYTES == 9_437_184 * 2
    # Per token: router 2*64*2048 plus 4 experts x 2 FLOP x 3 x 2048 x 1536.
    assert bench.FLOP_PER_TOKEN == 262_144 + 75_497_472
    assert bench.layer_bytes(40, 64) == 40 * 18_874_368 + 262_144 + 256 + 64 * 12_288
    assert bench.gateup_flops(4096) == 4 * 4096 * 2 * 3072 * 2048
    # FP8 experts: one byte per weight and a fp32 scale per 128 x 128 block
    # (gate and up: 2 x 12 x 16 blocks, down: 16 x 12).
    assert bench.FP8_GATEUP_W_BYTES + bench.FP8_DOWN_W_BYTES == 9_437_184 + (384 + 192) * 4
    # grouped kernels (N > 4): token codes and scales; streaming kernels: bf16 rows
    assert bench.fp8_gateup_bytes(40, 64) == 40 * 6_292_992 + 64 * (2048 + 64) + 256 * 3072
    assert bench.fp8_gateup_bytes(40, 4) == 40 * 6_292_992 + 4 * 4096 + 16 * 3072
    assert bench.fp8_down_bytes(40, 64) == 40 * 3_146_496 + 256 * (1536 + 48) + 256 * 8192


def _summary(N, A, ms, gu_ms):
    h = dict(N=N, active_experts=A, max_tokens_per_expert=17, ms_per_step=ms,
             tokens_per_s=N / (ms * 1e-3), layer_gbs=bench.layer_bytes(A, N) / (ms * 1e-3) / 1e9,
             layer_hbm_frac=0.1, layer_tflops=N * bench.FLOP_PER_TOKEN / (ms * 1e-3) / 1e12,
             layer_mfma_frac=0.1, kernel_ms=dict(gateup=gu_ms, down=0.05, route=0.01),
             gateup_gbs=bench.gateup_bytes(A, N) / (gu_ms * 1e-3) / 1e9,
             gateup_tflops=bench.gateup_flops(N) / (gu_ms * 1e-3) / 1e12)
    return h


def test_json_line_and_roofline_selection():
    args = bench.parse_args([])
    h = _summary(64, 40, 0.15, 0.09)
    p = _summary(4096, 52, 0.75, 0.4)
    line = bench.build_line(args, h, 1, p, dict(value=1.0, unit="tokens/s", cores=16,
                                               kind="oracle", sample="x"))
    json.dumps(line)
    assert line["metric"] == bench.METRIC and line["unit"] == "tokens/s"
    assert line["config"]["workload"] == "decode_n64" and line["config"]["N"] == 64
    r = line["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-12
    q = line["prefill"]["roofline"]
    assert q["bound"] == "mfma" and q["unit"] == "TFLOP/s" and q["peak"] == 2500.0
    # The bound follows the algorithmic intensity: 640 tokens on 48 experts
    # (about 53 FLOP/B) is HBM-bound although N > 512.
    assert bench.hbm_bound(_summary(640, 48, 0.22, 0.12))
    assert not bench.hbm_bound(_summary(16384, 44, 1.5, 0.8))
