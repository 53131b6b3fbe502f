"""Helpers shared by the GPU parity tests: move seeded workloads to the device, run the oracle on
the same inputs, and compare: decisions bit-exact away from near ties, probabilities within 1e-5
relative, attention outputs within 2e-2 absolute."""

import sys

import numpy as np
import torch

from oracle import accept as o_accept
from oracle import philox as o_philox

NEAR_TIE = 1e-6          # decisions closer than this to flipping are reported, not compared
P_REL = 1e-5             # p_tok / q_tok relative error (fp32)
ATTN_BF16_ABS = 2e-2     # attention output, bf16 path
ATTN_F32_ABS = 1e-5      # attention output, fp32 path


# What each parity check measured (name -> dict), printed in pytest's terminal summary so that a
# captured run still shows the error magnitudes and near-tie counts against the tolerances.
RESULTS = {}


def record(name, **values):
    RESULTS.setdefault(name, {}).update(values)


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(arr, dtype):
    """numpy float32 (bf16-representable when dtype is bf16) -> device tensor of `dtype`."""
    t = torch.from_numpy(np.ascontiguousarray(arr)).to("cuda")
    return t.to(dtype)


def logits_dtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def run_accept_gpu(w, seed=None, offset=None, draft=True, siblings="without_replacement"):
    import draft_verify_sampling_specv_amd as specv
    dt = logits_dtype(w)
    tl = dev(w.target_logits, dt)
    dl = dev(w.draft_logits, dt) if (draft and w.T > 0) else None
    tok = torch.from_numpy(np.ascontiguousarray(w.tokens, dtype=np.int32)).cuda()
    par = torch.from_numpy(np.ascontiguousarray(w.parent, dtype=np.int32)).cuda()
    r = specv.accept_resample(tl, dl, tok, par, w.T, w.seed if seed is None else seed,
                              w.offset if offset is None else offset, siblings=siblings)
    torch.cuda.synchronize()
    return {k: getattr(r, k).cpu().numpy() for k in ("accept_len", "out_tokens", "out_nodes", "p_tok", "q_tok")}


def run_accept_oracle(w, seqs=None, seed=None, offset=None, with_probs=True, siblings="without_replacement"):
    seed = w.seed if seed is None else seed
    offset = w.offset if offset is None else offset
    seqs = range(w.B) if seqs is None else seqs
    seqs = list(seqs)
    ua, ur = [], []
    for b in seqs:
        a_b, r_b = zip(*[o_philox.node_uniforms(seed, offset, b, v) for v in range(w.N1)])
        ua.append(list(a_b))
        ur.append(list(r_b))
    tl = np.asarray(w.target_logits[seqs], dtype=np.float64)
    dl = np.asarray(w.draft_logits[seqs], dtype=np.float64) if w.T > 0 else None
    return o_accept.accept_batch(tl, dl, w.tokens[seqs], w.parent[seqs], w.T, ua, ur, with_probs=with_probs,
                                 siblings=siblings)


def compare_accept(gpu, ora, seqs=None, check_probs=True, name=""):
    """Bit-exact accept_len / out_tokens / out_nodes outside near ties; p/q within P_REL."""
    seqs = list(range(len(ora["accept_len"]))) if seqs is None else list(seqs)
    near = 0
    bad = []
    for j, b in enumerate(seqs):
        if ora["margin"][j] < NEAR_TIE:
            near += 1
            continue
        same = (gpu["accept_len"][b] == ora["accept_len"][j]
                and np.array_equal(gpu["out_tokens"][b], ora["out_tokens"][j])
                and np.array_equal(gpu["out_nodes"][b], ora["out_nodes"][j]))
        if not same:
            bad.append((b, int(gpu["accept_len"][b]), int(ora["accept_len"][j]),
                        gpu["out_tokens"][b][:6].tolist(), ora["out_tokens"][j][:6].tolist(),
                        float(ora["margin"][j])))
    log(f"[{name}] sequences {len(seqs)}, near ties {near}, mismatches {len(bad)}")
    record(name, kind="accept", sequences=len(seqs), near_ties=near, mismatches=len(bad))
    assert not bad, f"[{name}] mismatches (b, gpu_len, oracle_len, gpu_tok, oracle_tok, margin): {bad[:5]}"
    if check_probs:
        for key in ("p_tok", "q_tok"):
            g = gpu[key][seqs].astype(np.float64)
            o = ora[key]
            assert np.array_equal(np.isnan(g), np.isnan(o)), f"[{name}] {key} NaN pattern differs"
            fin = ~np.isnan(o)
            if fin.any():
                rel = np.abs(g[fin] - o[fin]) / np.maximum(np.abs(o[fin]), 1e-300)
                log(f"[{name}] {key} max rel err {rel.max():.3e}")
                record(name, **{f"{key}_max_rel": float(rel.max())})
                assert rel.max() <= P_REL, f"[{name}] {key} rel err {rel.max()}"
    return near
