"""Build libspecv.so (HIP, gfx950) in-tree, and its bounds-checked debug twin.

    python draft_verify_sampling_specv_amd/build.py      (or __graft_entry__.build())

Every .hip file under csrc/ is compiled to an object with hipcc and the objects
are linked into draft_verify_sampling_specv_amd/libspecv.so.  Packed-fp32 ops
are disabled for all device code.  build(checked=True) compiles the same sources
with SPECV_CHECKED (every data-derived index range-checked, see common.h) as
relocatable device code, so that the kernels of all files share one record
word, into libspecv_checked.so.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libspecv.so")
LIB_CHECKED = os.path.join(PKG, "libspecv_checked.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src, build_dir=BUILD, extra=()):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature; drop that noise
    err = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose=True, checked=False):
    build_dir = os.path.join(BUILD, "checked") if checked else BUILD
    lib = LIB_CHECKED if checked else LIB
    extra = ("-DSPECV_CHECKED", "-fgpu-rdc") if checked else ()
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, extra), srcs))
    tmp = lib + ".tmp"
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(["-fgpu-rdc", "--hip-link"] if checked else []),
            *objs, "-o", tmp]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build()
    build(checked=True)
