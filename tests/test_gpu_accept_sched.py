"""Accept / resample under every schedule: the result must not depend on when the workgroups that
share a sequence run.

A workgroup waits for a teammate's values for at most a budget (SPECV_ACCEPT_WAIT_US) and then
computes them itself.  With a budget of 0 almost every value not yet published when first read
is computed on the owner's behalf; the outputs must stay bit-identical to the default run and
to the oracle.  The same holds with another stream holding compute units, and for a call
captured in a graph and replayed (each launch takes a new epoch from the workspace).

The chunk statistics run either inside the team kernel or as a launch of their own before it
(SPECV_ACCEPT_SPLIT; by default the split where each workgroup would get many items): the wait
tests pin the team kernel's own statistics phase (SPECV_ACCEPT_SPLIT=0), and the two forms must
give the same bits on every configuration.
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_common import compare_accept, dev, log, logits_dtype, record, run_accept_oracle

pytestmark = pytest.mark.gpu

KEYS = ("accept_len", "out_tokens", "out_nodes", "p_tok", "q_tok")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _specv():
    import draft_verify_sampling_specv_amd as specv
    return specv


def _inputs(w):
    dt = logits_dtype(w)
    tl = dev(w.target_logits, dt)
    dl = dev(w.draft_logits, dt) if w.T > 0 else None
    tok = torch.from_numpy(np.ascontiguousarray(w.tokens, dtype=np.int32)).cuda()
    par = torch.from_numpy(np.ascontiguousarray(w.parent, dtype=np.int32)).cuda()
    return tl, dl, tok, par


def _run(w, inputs, bufs, offset=None):
    specv = _specv()
    tl, dl, tok, par = inputs
    r = specv.accept_resample(tl, dl, tok, par, w.T, w.seed, w.offset if offset is None else offset,
                              buffers=bufs)
    torch.cuda.synchronize()
    return {k: getattr(r, k).cpu().numpy().copy() for k in KEYS}


def _counters(bufs):
    """(batches of chunk statistics, range partials) computed on a teammate's behalf so far."""
    c = bufs.workspace[8:24].view(torch.int64).cpu().numpy()
    return int(c[0]), int(c[1])


def _same(a, b, name):
    for k in KEYS:
        np.testing.assert_array_equal(a[k], b[k], err_msg=f"[{name}] {k}")


CASES = {
    "chain": lambda: workloads.chain_config(T=1.0),
    "chain-greedy": lambda: workloads.chain_config(T=0.0),
    "eagle": workloads.eagle_config,
    "stress": workloads.stress_config,
    "ptd": workloads.ptd_config,
}


@pytest.mark.parametrize("name", list(CASES))
def test_accept_exact_when_every_wait_gives_up(name, monkeypatch):
    specv = _specv()
    w = CASES[name]()
    inputs = _inputs(w)
    log(f"accept {name}: default wait, then a wait budget of 0")
    b0 = specv.AcceptBuffers.allocate(w.B, w.N1, w.V, logits_dtype(w), "cuda")
    ref = _run(w, inputs, b0)
    monkeypatch.setenv("SPECV_ACCEPT_WAIT_US", "0")
    monkeypatch.setenv("SPECV_ACCEPT_SPLIT", "0")
    b1 = specv.AcceptBuffers.allocate(w.B, w.N1, w.V, logits_dtype(w), "cuda")
    outs = [_run(w, inputs, b1) for _ in range(3)]
    items, parts = _counters(b1)
    log(f"[{name}] wait 0: {items} statistics batches and {parts} range partials computed for a teammate")
    record(f"wait0-{name}", kind="schedule", recomputed_stat_batches=items, recomputed_partials=parts)
    for o in outs:
        _same(ref, o, name)
    if name in ("chain", "eagle", "ptd"):
        compare_accept(outs[0], run_accept_oracle(w), name=f"wait0-{name}")


SPLIT_CASES = dict(CASES, tiny=lambda: workloads.tiny_chain_trials(10_000),
                   # vocabularies that are no multiple of the 16-byte vector: the element-load path
                   **{"oddV-f32": lambda: workloads.random_case(501, 40, 17, 20011, 0.9, dtype="f32"),
                      "oddV-bf16": lambda: workloads.random_case(502, 24, 23, 65537, 1.2, dtype="bf16"),
                      "oddV-greedy": lambda: workloads.random_case(503, 24, 23, 65537, 0.0, dtype="bf16")})


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_accept_split_statistics_launch_gives_the_same_bits(name, monkeypatch):
    """Phase 1 as its own launch (one wave per item over the whole device) or inside the team
    kernel: the same arithmetic on the same items, so identical outputs, call after call."""
    specv = _specv()
    w = SPLIT_CASES[name]()
    inputs = _inputs(w)
    bufs = specv.AcceptBuffers.allocate(w.B, w.N1, w.V, logits_dtype(w), "cuda")
    for i in range(2):
        monkeypatch.setenv("SPECV_ACCEPT_SPLIT", "0")
        fused = _run(w, inputs, bufs, offset=w.offset + i)
        monkeypatch.setenv("SPECV_ACCEPT_SPLIT", "1")
        split = _run(w, inputs, bufs, offset=w.offset + i)
        _same(fused, split, f"split-{name}-{i}")
    log(f"[{name}] statistics launched apart and inside the team kernel: identical outputs")


def test_accept_wait_zero_takes_the_recompute_paths(monkeypatch):
    """On a team of several workgroups, a budget of 0 must actually exercise both paths."""
    specv = _specv()
    w = workloads.eagle_config()          # B = 16: teams of 16 workgroups
    inputs = _inputs(w)
    monkeypatch.setenv("SPECV_ACCEPT_WAIT_US", "0")
    monkeypatch.setenv("SPECV_ACCEPT_SPLIT", "0")
    bufs = specv.AcceptBuffers.allocate(w.B, w.N1, w.V, logits_dtype(w), "cuda")
    for i in range(5):
        _run(w, inputs, bufs, offset=w.offset + i)
    items, parts = _counters(bufs)
    log(f"eagle, wait 0, 5 calls: {items} statistics batches, {parts} partials recomputed")
    assert items > 0 and parts > 0


def test_accept_exact_beside_a_concurrent_stream():
    """Another stream keeps compute units busy while accept runs; outputs stay exact."""
    specv = _specv()
    side = torch.cuda.Stream()
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    bm = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16).contiguous()
    for name in ("chain", "eagle"):
        w = CASES[name]()
        inputs = _inputs(w)
        bufs = specv.AcceptBuffers.allocate(w.B, w.N1, w.V, logits_dtype(w), "cuda")
        ref = _run(w, inputs, bufs)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            for _ in range(12):
                torch.matmul(a, bm)
        outs = []
        results = []
        for i in range(6):
            r = specv.accept_resample(*inputs[:2], inputs[2], inputs[3], w.T, w.seed, w.offset, buffers=bufs)
            results.append({k: getattr(r, k).clone() for k in KEYS})
        torch.cuda.synchronize()
        outs = [{k: v.cpu().numpy() for k, v in res.items()} for res in results]
        items, parts = _counters(bufs)
        log(f"[{name}] beside a busy stream: {items} statistics batches, {parts} partials recomputed")
        record(f"concurrent-{name}", kind="schedule", recomputed_stat_batches=items, recomputed_partials=parts)
        for o in outs:
            _same(ref, o, f"concurrent-{name}")
        compare_accept(outs[-1], run_accept_oracle(w), name=f"concurrent-{name}")


@pytest.mark.parametrize("split", ["0", "1"])
def test_accept_graph_replays_take_new_epochs(split, monkeypatch):
    """One captured call replayed with new logits each time matches the eager call every time, with
    the statistics inside the team kernel (one launch captured) and as a launch of their own (two)."""
    monkeypatch.setenv("SPECV_ACCEPT_SPLIT", split)
    specv = _specv()
    base = workloads.eagle_config()
    dt = logits_dtype(base)
    tl, dl, tok, par = _inputs(base)
    bufs = specv.AcceptBuffers.allocate(base.B, base.N1, base.V, dt, "cuda")
    specv.accept_resample(tl, dl, tok, par, base.T, base.seed, base.offset, buffers=bufs)     # warm
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        specv.accept_resample(tl, dl, tok, par, base.T, base.seed, base.offset, buffers=bufs)
    torch.cuda.synchronize()
    eager = specv.AcceptBuffers.allocate(base.B, base.N1, base.V, dt, "cuda")
    for rep in range(4):
        w = workloads.eagle_config(seed_base=3000 + 101 * rep) if rep else base
        tl.copy_(dev(w.target_logits, dt))
        dl.copy_(dev(w.draft_logits, dt))
        tok.copy_(torch.from_numpy(np.ascontiguousarray(w.tokens, dtype=np.int32)).cuda())
        par.copy_(torch.from_numpy(np.ascontiguousarray(w.parent, dtype=np.int32)).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {k: getattr(bufs.result, k).cpu().numpy().copy() for k in KEYS}
        want = _run(base, (tl, dl, tok, par), eager)
        _same(want, got, f"graph-replay{rep}-split{split}")
        log(f"graph replay {rep} (split {split}): identical to the eager call")
