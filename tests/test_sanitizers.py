"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The library's host half -- the block pool, the decode planner, the
  argument checks of every entry point -- built from the product sources
  with the sanitizers on the host side only (`-Xarch_host`; the gfx950
  device code is compiled as usual and never launched) and linked into
  tests/sanitize/host_abi_driver.cpp, which drives random pool scripts
  against its own reference counts, a grid of ~45,000 planner argument
  sets and the rejection paths of every device entry point.
* The CPU oracle built with gcc's sanitizers and run through every pin of
  tests/pins.py in a subprocess (the ASan runtime preloaded into Python).

Any sanitizer report fails the run (halt_on_error, no recovery)."""
import concurrent.futures
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_192_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")

pytestmark = pytest.mark.slow


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_library_host_code_under_asan_and_ubsan(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    flags = ["-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC] + san
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    srcs.append(os.path.join(ROOT, "tests", "sanitize", "host_abi_driver.cpp"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC] + flags + ["-c", src, "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "host_abi_driver")
    _run([HIPCC, "--offload-arch=gfx950"] + san[:4] + ["-o", exe] + objs)
    r = _run([exe], env=SAN_ENV, timeout=600)
    assert r.stdout.strip().endswith("ok"), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libpa_oracle_san.so")
    _run(["gcc", "-O1", "-g", "-std=gnu11", "-fopenmp", "-fPIC", "-shared", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-o", lib,
          os.path.join(ROOT, "oracle", "pa_oracle.c"), "-lm"])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(SAN_ENV, LD_PRELOAD=asan, OMP_NUM_THREADS="4")
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import oracle, pins\n"
            "with oracle.use_library(%r):\n"
            "    for p in pins.ALL_PINS: p()\n"
            "print('pins ok', len(pins.ALL_PINS))\n" % (ROOT, os.path.join(ROOT, "tests"), lib))
    r = _run([sys.executable, "-c", code], env=env, timeout=900)
    assert "pins ok" in r.stdout, r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
