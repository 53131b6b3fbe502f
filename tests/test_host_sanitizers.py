"""Host code of the library under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Every source of the library is compiled with the sanitizers on its host code only (each
-fsanitize= behind -Xarch_host; the device code is built as usual and never runs here), linked
with tests/host_abi_sanitize.cpp, and run: every entry point is called with invalid or empty
arguments and must return its documented status without launching anything, with no sanitizer
report.  Skipped where hipcc is not installed.
"""

import glob
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xarch_host", "-fno-omit-frame-pointer",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN, f"-I{os.path.join(ROOT, 'include')}"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_entry_points_reject_bad_arguments_under_sanitizers():
    srcs = sorted(glob.glob(os.path.join(ROOT, "draft_verify_sampling_specv_amd", "csrc", "*.hip")))
    srcs.append(os.path.join(ROOT, "tests", "host_abi_sanitize.cpp"))
    tmp = tempfile.mkdtemp(prefix="specv_san_")
    try:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            r = subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True, timeout=600)
            assert r.returncode == 0, f"{src}:\n{r.stderr[-3000:]}"
            return obj

        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            objs = list(ex.map(compile_one, srcs))
        exe = os.path.join(tmp, "abi_san")
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, "-o", exe], capture_output=True, text=True,
                           timeout=600)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        out = r.stdout + r.stderr
        assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
        assert r.returncode == 0 and "ok: 0 failing checks" in out, out[-4000:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
