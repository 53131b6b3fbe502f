"""The bounds-checked build (libspecv_checked.so, compiled with SPECV_CHECKED).

In that build every kernel access whose index is derived from input data -- parent and token
values, context lengths, accepted node ids, frontier entries -- is range-checked; an index out of
range is recorded and replaced by 0, so the access stays in its buffer.  This test runs, in a child
process on that library, the GPU tests that drive the kernels with arbitrary shapes and hostile
inputs: random trees and chains up to 1024 nodes, invalid parent arrays, tokens and context lengths,
random accepted paths for the cache commit, random expansion levels, random layer trees, and the
accept call with its statistics inside the team kernel and as a launch of their own.  Each
must pass against the oracle as on the product library, and leave the bounds record clear (the
conftest fixture reads it after every GPU test under SPECV_LIBRARY=libspecv_checked.so).
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHECKED = os.path.join(ROOT, "draft_verify_sampling_specv_amd", "libspecv_checked.so")

FILES = ["tests/test_gpu_parity.py", "tests/test_gpu_kv_commit.py", "tests/test_gpu_tree_expand.py",
         "tests/test_gpu_layer.py", "tests/test_gpu_limits.py", "tests/test_gpu_accept_sched.py"]
SELECT = ("random or invalid or tiny or mask or short_context or jumps or empty or replays or draft_equals "
          "or long_path or after_gpu_accept or ties or max_nodes or split_statistics")


@pytest.mark.gpu
def test_checked_build_keeps_every_data_derived_index_in_range():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(CHECKED), "libspecv_checked.so not built"
    env = dict(os.environ, SPECV_LIBRARY="libspecv_checked.so")
    cmd = [sys.executable, "-u", "-m", "pytest", "-x", "-q", "-m", "gpu", "-p", "no:cacheprovider",
           *FILES, "-k", SELECT]
    print("child:", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = r.stdout[-4000:] + "\n" + r.stderr[-2000:]
    print(tail)
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and " failed" not in r.stdout, tail
