"""The C ABI's host-side code under AddressSanitizer and UBSan (CPU only).

The library is rebuilt with the sanitizers on its host code (each
`-fsanitize=` behind `-Xarch_host`; device code is unchanged) and a C++
driver (tests/sanitize/abi_checks.cpp) exercises every argument check, the
N = 0 no-ops and the workspace size arithmetic up to the largest N.  None of
those paths makes a HIP call, so no GPU is needed; any sanitizer report or
failed check fails the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "biased_sigmoid_top_amd", "csrc")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r


def test_abi_checks_under_address_and_ub_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    common = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              f"-I{os.path.join(ROOT, 'include')}"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    lib = tmp_path / "liblfm_moe_san.so"
    _run([hipcc, *common, *san, "-fPIC", "-shared", *srcs, "-o", str(lib)], timeout=900)
    exe = tmp_path / "abi_checks"
    _run([hipcc, *common, *san, os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp"),
          f"-L{tmp_path}", "-llfm_moe_san", f"-Wl,-rpath,{tmp_path}", "-o", str(exe)], timeout=300)
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([str(exe)], env=env, timeout=120)
    assert "abi checks ok" in r.stdout
