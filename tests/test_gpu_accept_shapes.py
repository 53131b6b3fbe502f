"""Accept over many batch shapes: team sizes from 1 to 64 workgroups per sequence, several sequences
per team (B above the team count), chains and trees, bf16 and fp32, and wait budgets of 0 and the
default -- the cross-workgroup exchange (statistics words, range partials, the launch epoch) under
every grid the launch planner makes.  Bit-exact against the oracle outside near ties."""

import numpy as np
import pytest
import torch

import workloads
from gpu_common import compare_accept, log, run_accept_gpu, run_accept_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# (B, n1, V, T, dtype): B 1 .. 600 covers teams of 64 down to one workgroup per sequence and
# several sequences per team; V spans one to many statistics chunks, with ragged tails
SHAPES = [
    (1, 9, 50000, 1.0, "bf16"),
    (3, 17, 20000, 0.8, "f32"),
    (5, 33, 9001, 1.2, "bf16"),
    (7, 6, 70001, 1.0, "f32"),
    (40, 5, 3000, 1.0, "bf16"),
    (97, 9, 2049, 0.7, "f32"),
    (256, 4, 1000, 1.0, "bf16"),
    (300, 6, 800, 1.5, "f32"),
    (600, 3, 257, 1.0, "bf16"),
    (33, 65, 4096, 1.0, "bf16"),
]


@pytest.mark.parametrize("wait", ["default", "0"])
def test_accept_over_batch_shapes(wait, monkeypatch):
    if wait == "0":
        monkeypatch.setenv("SPECV_ACCEPT_WAIT_US", "0")
    rng = np.random.default_rng(77 if wait == "0" else 78)
    for i, (B, n1, V, T, dtype) in enumerate(SHAPES):
        mc = 1 if i % 3 == 0 else 3            # chains and trees
        w = workloads.random_case(int(rng.integers(1 << 30)), B, n1, V, T, dtype=dtype, max_children=mc)
        w.seed, w.offset = int(rng.integers(1 << 62)), int(rng.integers(1 << 40))
        log(f"accept shapes (wait {wait}): B={B} N1={n1} V={V} T={T} {dtype} children<={mc}")
        compare_accept(run_accept_gpu(w), run_accept_oracle(w), name=f"shape{i}-wait{wait}")
