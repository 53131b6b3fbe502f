"""The streaming-read probe (specv_read_probe, the read-ceiling measurement of bench.py): every
workgroup reads exactly its slice of the buffer once.  Each workgroup's sink word is the XOR of
the 32-bit words it read, so the words are checked against the same fold done on the host, for a
buffer that divides evenly among the workgroups and for one that leaves a ragged last slice."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nvec", [512 * 64, 512 * 37 + 5, 7])
def test_read_probe_reads_each_slice_once(nvec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verify_sampling_specv_amd as specv
    nb = int(specv.lib.specv_read_probe_sink_words())
    rng = np.random.default_rng(5)
    words = rng.integers(0, 2**32, size=4 * nvec, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
    specv.read_probe(buf, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    per = (nvec + nb - 1) // nb                  # 16-byte vectors per workgroup
    for b in range(nb):
        lo, hi = min(b * per, nvec), min(b * per + per, nvec)
        want = np.bitwise_xor.reduce(words[4 * lo:4 * hi]) if hi > lo else np.uint32(0)
        assert got[b] == want, f"workgroup {b}: {got[b]:#x} != {int(want):#x}"
