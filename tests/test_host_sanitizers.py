"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (host side only;
the device code is built as usual), driven by tests/host_sanitize.cpp with no GPU work: planning
over a grid of valid and invalid descriptors, plan info, pieces and workspace sizes, the argument
errors of every entry point, the two-strand schedule and the error strings. The objects are cached
under _build/sanitize by the hash of their sources and flags."""
import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "comm_overlap_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["plan.cpp", "strands.cpp", "runtime.cpp", "static_scratch.cpp", "gemm.hip", "attn.hip", "attn_bwd.hip"]
# -fsanitize applies to the host pass only (each behind -Xarch_host); the device code is built as the
# library builds it
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
FLAGS = ["--offload-arch=gfx950", "-x", "hip", "-O3", "-g", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN]

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _compile(path):
    text = open(path, "rb").read()
    deps = b"".join(open(os.path.join(d, f), "rb").read() for d in (CSRC, INCLUDE)
                    for f in sorted(os.listdir(d)) if f.endswith((".h", ".hpp")))
    key = hashlib.sha256(text + deps + " ".join(FLAGS).encode()).hexdigest()[:16]
    obj = os.path.join(OUT, f"{os.path.basename(path)}.{key}.o")
    if not os.path.exists(obj):
        r = subprocess.run([HIPCC, *FLAGS, "-c", path, "-o", obj + ".tmp"], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        os.replace(obj + ".tmp", obj)
    return obj


def test_host_code_under_address_and_undefined_behaviour_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    paths = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(ROOT, "tests", "host_sanitize.cpp")]
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, paths))
    exe = os.path.join(OUT, "host_sanitize")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.startswith("ok:"), r.stdout
