"""The exactness rule, read empirically on the GPU ([SD-EAGLE] "The Exactness Rule"; [SD-review]
section 2, "Mathematical guarantee"): the first token a step emits -- the accepted draft token, or
the replacement drawn from the residual after a rejection -- is distributed exactly as p, the
target's distribution at the root, whatever the draft.  Over 10^6 independent trials of the tiny
chain (K = 4, V = 1000, fp32, T = 1; fresh draft tokens drawn from q per trial, fresh uniforms per
trial) the total-variation distance between the emitted tokens' empirical law and p must stay
below 0.01 (about 0.007 is the sampling noise of 10^6 draws from this p; an inexact rule, e.g. one
that drew the replacement from p instead of the residual, lands far above)."""

import numpy as np
import pytest
import torch

import workloads
from gpu_common import log, record

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_first_emitted_token_follows_p_over_a_million_trials():
    import draft_verify_sampling_specv_amd as specv
    base = workloads.tiny_chain_trials(1)                  # the configuration's logits
    t1 = torch.from_numpy(np.array(base.target_logits[0], copy=True)).cuda()     # [K+1][V] fp32
    d1 = torch.from_numpy(np.array(base.draft_logits[0], copy=True)).cuda()
    n1, V = t1.shape
    K = n1 - 1
    trials, per_call = 1_000_000, 100_000
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261)
    q = torch.softmax(d1[:K].double(), dim=-1)              # the draft rows that propose positions 1..K
    target = t1.unsqueeze(0).expand(per_call, n1, V).contiguous()
    draft = d1.unsqueeze(0).expand(per_call, n1, V).contiguous()
    parent = torch.tensor(np.asarray(workloads.chain_parent(per_call, K)), dtype=torch.int32, device="cuda")
    counts = torch.zeros(V, dtype=torch.float64, device="cuda")
    bufs = specv.AcceptBuffers.allocate(per_call, n1, V, torch.float32, "cuda")
    for c in range(trials // per_call):
        tokens = torch.empty((per_call, n1), dtype=torch.int32, device="cuda")
        tokens[:, 0] = int(base.tokens[0, 0])
        for j in range(K):
            tokens[:, j + 1] = torch.multinomial(q[j], per_call, replacement=True, generator=gen).to(torch.int32)
        r = specv.accept_resample(target, draft, tokens, parent, 1.0, seed=777, offset=c, buffers=bufs,
                                  with_probs=False)
        counts += torch.bincount(r.out_tokens[:, 0].long(), minlength=V).double()
    torch.cuda.synchronize()
    emp = (counts / trials).cpu().numpy()
    t0 = base.target_logits[0, 0].astype(np.float64)
    p = np.exp(t0 - t0.max())
    p /= p.sum()
    tv = 0.5 * float(np.abs(emp - p).sum())
    noise = 0.5 * float(np.sum(np.sqrt(2 * p * (1 - p) / (np.pi * trials))))
    log(f"first emitted token over {trials} trials: TV to p = {tv:.5f} (sampling noise about {noise:.5f})")
    record("exactness-tv", kind="tv", trials=trials, tv=tv, expected_noise=noise)
    assert tv < 0.01
