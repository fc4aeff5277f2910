"""CPU-side checking aids: the oracle and the host side of the C ABI built
with AddressSanitizer and UndefinedBehaviorSanitizer, driven on small and
edge-case shapes (tests/sanitize/*_driver.*).  Sanitizers apply to host code
only: the HIP sources are compiled with the sanitizer flags on the host pass
alone, and no kernel is launched."""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-fopenmp", os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "dsa_oracle.c"), "-lm", "-o", exe])
    r = _run([exe], env=dict(ENV, OMP_NUM_THREADS="4"))
    assert "oracle driver: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_abi_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-strict-aliasing",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include"),
             "-I", os.path.join(ROOT, "long_context_sparse_dsa_amd", "csrc")]
    srcs = sorted(glob.glob(os.path.join(ROOT, "long_context_sparse_dsa_amd", "csrc", "*.hip")))
    srcs.append(os.path.join(SAN, "abi_driver.cpp"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *flags, "-c", src, "-o", obj])
        return obj
    with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_san")
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", *objs, "-o", exe])
    # the HIP runtime keeps allocations alive until exit: leaks are not checked here
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=0"))
    assert "abi driver: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
