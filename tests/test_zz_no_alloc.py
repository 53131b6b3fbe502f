"""The allocation-free accept entry point (specv_accept_resample_rule_noalloc, workspace built into
the library) against the entry point with a caller's workspace: identical outputs on two calls in
a row, the second with a smaller input, and the size limit reported as an error."""

import numpy as np
import pytest
import torch

import workloads
from gpu_common import dev, log, logits_dtype

pytestmark = pytest.mark.gpu

KEYS = ("accept_len", "out_tokens", "out_nodes", "p_tok", "q_tok")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(w):
    dt = logits_dtype(w)
    tl = dev(w.target_logits, dt)
    dl = dev(w.draft_logits, dt) if w.T > 0 else None
    tok = torch.from_numpy(np.ascontiguousarray(w.tokens, dtype=np.int32)).cuda()
    par = torch.from_numpy(np.ascontiguousarray(w.parent, dtype=np.int32)).cuda()
    return tl, dl, tok, par


def _both(w, siblings="without_replacement"):
    import draft_verify_sampling_specv_amd as specv
    tl, dl, tok, par = _inputs(w)
    a = specv.accept_resample(tl, dl, tok, par, w.T, w.seed, w.offset, siblings=siblings)
    torch.cuda.synchronize()
    want = {k: getattr(a, k).cpu().numpy().copy() for k in KEYS}
    b = specv.accept_resample_noalloc(tl, dl, tok, par, w.T, w.seed, w.offset, siblings=siblings)
    torch.cuda.synchronize()
    got = {k: getattr(b, k).cpu().numpy().copy() for k in KEYS}
    return want, got


def _same(want, got, name):
    for k in KEYS:
        np.testing.assert_array_equal(got[k], want[k], err_msg=f"[{name}] {k}")


def test_noalloc_matches_workspace_entry_on_two_calls_second_smaller():
    cases = [("eagle B=16 N=61 V=128256 bf16", workloads.eagle_config()),
             ("chain B=32 K=5 V=32000 bf16", workloads.chain_config(T=1.0))]
    for name, w in cases:
        log(f"no-alloc accept: {name}")
        want, got = _both(w)
        _same(want, got, name)
    # a smaller call again, fp32, and a greedy one (the array keeps the previous calls' words)
    w = workloads.random_case(77, 5, 9, 3001, 0.8)
    want, got = _both(w, siblings="iid")
    _same(want, got, "random fp32 B=5 N=9 V=3001")
    w = workloads.chain_config(T=0.0)
    want, got = _both(w)
    _same(want, got, "chain greedy")


def test_noalloc_rejects_calls_beyond_its_workspace():
    import draft_verify_sampling_specv_amd as specv
    B, n1, V = 256, 129, 262144
    need = specv.accept_workspace_bytes(B, n1 - 1, V, torch.float32)
    assert need > (8 << 20)
    # shapes only: the size check comes before any pointer is read, so views of a small buffer do
    tl = torch.zeros(1, dtype=torch.float32, device="cuda").expand(B, n1, V)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda").expand(B, n1)
    res = specv.AcceptResult(*(torch.empty(1, device="cuda") for _ in range(5)))
    status = specv.lib.specv_accept_resample_rule_noalloc(
        tl.data_ptr(), tl.data_ptr(), 0, tok.data_ptr(), tok.data_ptr(), B, n1 - 1, V, 1.0, 0, 0, 0,
        res.accept_len.data_ptr(), res.out_tokens.data_ptr(), res.out_nodes.data_ptr(), None, None, None)
    assert status == 3, specv.lib.specv_last_error()
