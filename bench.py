"""Benchmark of the verify step on one MI355X.

One step = the whole hot path over one batch of the chain workload (B=32, K=5, V=32000 bf16
logits, T=1; attention over a 2048-token bf16 KV cache, 32 query / 8 KV heads, head size 128):
  specv_build_tree_mask -> specv_tree_attn_verify (one layer) -> specv_accept_resample.
value = draft positions verified per second = B*K / step time.  Inputs are resident in HBM and
rotate over enough sets (> 2 x 256 MB) that the Infinity Cache cannot serve them.

Prints ONE JSON line.  Extra legs:
  roofline      attention call (HBM-bound here): algorithmic bytes / mean call time (HIP events
                on the launch stream), against the nominal 8 TB/s and against the read ceiling
                measured in the same run (specv_read_probe over 1 GiB); the accept call's figure
                is reported beside it;
  cpu_baseline  the oracle (numpy fp64) on a bounded sample of the same workload, host cores.

  verify_layer  one whole target layer over the same 192 rows (specv_verify_layer): its time,
                the attention call's share of it, and the weight-streaming rate of the rest.
  configs       every configuration of the workload list (tiny, chain, chain-greedy, eagle,
                stress, ptd): us per kernel, HBM fractions of accept and attention, MFMA fraction of
                attention, positions/s accept-only and verify, alpha and the expected tokens per
                step against the measured mean.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-layer] [--no-configs]
                  [--config NAME] [--copy-probe]
--copy-probe only runs a device-to-device copy of known size (to calibrate HBM byte counters).
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

METRIC = "draft positions verified/s (B=32,V=32k,K=5) + % of MI355X HBM roofline"
HBM_PEAK_GBS = 8000.0
B, K, V, T = 32, 5, 32000, 1.0
HQ, HKV, D, CTX = 32, 8, 128, 2048
ACCEPT_SETS = 24          # 24 x 22.5 MB of logits
ATTN_SETS = 3             # 3 x 269 MB of KV cache


# configurations: accept generator, attention generator, draft positions per sequence, description
CONFIGS = {
    "tiny": "tiny oracle case: chain K=4, V=1000 fp32, 10^4 trials; six-node tree attention, 4 heads, D=64, ctx 128, fp32",
    "chain": "chain B=32, K=5, V=32000 bf16, T=1; attention ctx 2048, 32/8 heads, D=128 bf16",
    "chain-greedy": "chain B=32, K=5, V=32000 bf16, T=0 (greedy)",
    "eagle": "EAGLE-style tree B=16, 60 nodes (top-3, depth 6), V=128256 bf16, T=0.7; attention ctx 4096, 64/8 heads, D=128",
    "stress": "low-acceptance chain B=64, K=8, V=151936 fp32, T=1.5; attention ctx 1024, 40/8 heads, D=128 bf16",
    "ptd": "PTD-style tree B=4, 64 nodes (<=4 children, depth <=8), V=128256 bf16, T=1; attention ctx 32768, 64/8 heads",
}
MFMA_PEAK_TFLOPS = 2500.0

# HBM traffic of the dominant kernel (attn_decode_kernel<128, 8, 1>) per call on this workload, from
# two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE, KiB per dispatch), each scaled by what the same
# counter reads for a 256 MiB device-to-device copy (FETCH_SIZE 131084.5 KiB -> x1.99981,
# WRITE_SIZE 262144.0 KiB -> x1.0).  Summaries and commands: profiles/chain_step_pmc.md.
# Valid only for the kernel sources it was measured on (their SHA-256 below); null otherwise.
ATTN_TRAFFIC = {
    "sources": ["draft_verify_sampling_specv_amd/csrc/attn_decode.hip",
                "draft_verify_sampling_specv_amd/csrc/attn_common.h",
                "draft_verify_sampling_specv_amd/csrc/common.h",
                "draft_verify_sampling_specv_amd/csrc/kernels.h"],
    "sha256": "39415d793b42e2def947e52b93f1c8aa32691554e646b07d440cbe75d69dcf9e",
    "fetch_kib": 132320.6, "write_kib": 1584.0, "fetch_scale": 262144.0 / 131084.5, "write_scale": 1.0,
}

# The same for the sampled accept kernel (accept_kernel<bf16, sampled>) on this workload: the
# statistics pass reads the 22.5 MB of rows once, the draw re-reads the end node's rows (about
# 4 MB), and the writes are mostly register spill stores.
ACCEPT_TRAFFIC = {
    "sources": ["draft_verify_sampling_specv_amd/csrc/accept.hip",
                "draft_verify_sampling_specv_amd/csrc/common.h",
                "draft_verify_sampling_specv_amd/csrc/kernels.h"],
    "sha256": "6984583b9eb650fab22f538ef373df6d8748b611f31f6b2a18fb7349f15c67cb",
    "fetch_kib": 13200.9, "write_kib": 2164.0, "fetch_scale": 262144.0 / 131084.5, "write_scale": 1.0,
}


def traffic_bytes(t):
    import hashlib
    h = hashlib.sha256()
    for f in t["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != t["sha256"]:
        return None
    return (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024.0


def attn_traffic_bytes():
    return traffic_bytes(ATTN_TRAFFIC)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline leg")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--no-layer", action="store_true", help="skip the one-layer measurement")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration legs")
    ap.add_argument("--config", default=None, choices=sorted(CONFIGS),
                    help="measure every kernel on one configuration (prints a per-config JSON line "
                         "instead of the headline line)")
    return ap.parse_args()


def copy_probe(torch):
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": n, "launches": 10}))


def accept_bytes(n1, n_internal, V, elem):
    """Algorithmic HBM bytes of one accept call: every target row and the draft rows of internal
    nodes once, plus the tiny per-node inputs and outputs."""
    return B * (n1 + n_internal) * V * elem + B * n1 * 4 * 6 + B * 4


def attn_bytes(ctx, n1):
    """K and V of the context and of the tree entries once, Q in and O out (bf16), LSE out."""
    kv = 2 * B * HKV * (ctx + n1) * D * 2
    qo = 2 * B * n1 * HQ * D * 2 + B * n1 * HQ * 4
    return kv + qo


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verify step shards by sequence and KV head with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import draft_verify_sampling_specv_amd as specv
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(torch)
        return
    if args.config:
        print(json.dumps(measure_config(args.config, args, torch, specv, workloads)))
        return

    n1 = K + 1
    # ---- inputs (seeded, synthetic) resident in HBM
    t0 = time.time()
    acc_sets = []
    for s in range(ACCEPT_SETS):
        w = workloads.chain_config(T=T, seed_base=2000 + 17 * s)
        acc_sets.append(dict(
            target=torch.from_numpy(w.target_logits).cuda().to(torch.bfloat16),
            draft=torch.from_numpy(w.draft_logits).cuda().to(torch.bfloat16),
            tokens=torch.from_numpy(w.tokens).cuda(), parent=torch.from_numpy(w.parent).cuda(),
            w=w if s == 0 else None))
    greedy = workloads.chain_config(T=0.0)
    g_target = torch.from_numpy(greedy.target_logits).cuda().to(torch.bfloat16)
    g_tokens = torch.from_numpy(greedy.tokens).cuda()
    a0 = workloads.chain_attention(B=B)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    attn_sets = []
    for s in range(ATTN_SETS):
        if s == 0:
            q = torch.from_numpy(a0.q).cuda().to(torch.bfloat16)
            kc = torch.from_numpy(a0.k_cache).cuda().to(torch.bfloat16)
            vc = torch.from_numpy(a0.v_cache).cuda().to(torch.bfloat16)
        else:
            shape = tuple(a0.k_cache.shape)
            q = torch.randn(a0.q.shape, generator=gen, device="cuda").to(torch.bfloat16)
            kc = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
            vc = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
        attn_sets.append((q, kc, vc))
    ctx_len = torch.full((B,), CTX, dtype=torch.int32, device="cuda")
    parent = acc_sets[0]["parent"]
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s")

    # ---- preallocated outputs and workspaces (nothing is allocated inside the timed region)
    mask_out = (torch.empty((B, n1, 1), dtype=torch.int32, device="cuda"),
                torch.empty((B, n1), dtype=torch.int32, device="cuda"),
                torch.empty((B,), dtype=torch.int32, device="cuda"))
    abuf = specv.AttnBuffers.allocate(attn_sets[0][0], attn_sets[0][1])
    cbuf = specv.AcceptBuffers.allocate(B, n1, V, torch.bfloat16, "cuda")
    gbuf = specv.AcceptBuffers.allocate(B, n1, V, torch.bfloat16, "cuda")

    def step(i):
        a = acc_sets[i % ACCEPT_SETS]
        q, kc, vc = attn_sets[i % ATTN_SETS]
        mask, _, _ = specv.build_tree_mask(parent, out=mask_out)
        specv.tree_attn_verify(q, kc, vc, ctx_len, mask, buffers=abuf)
        specv.accept_resample(a["target"], a["draft"], a["tokens"], a["parent"], T, seed=1234, offset=i,
                              buffers=cbuf)

    def timed(fn, n):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(n):
            fn(i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n   # ms per call

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_step = timed(step, args.steps)

    # ---- per-call times (same stream, same rotation), for the rooflines
    mask_now = specv.build_tree_mask(parent, out=mask_out)[0]
    ms_attn = timed(lambda i: specv.tree_attn_verify(*attn_sets[i % ATTN_SETS], ctx_len, mask_now,
                                                     buffers=abuf), args.steps)
    ms_accept = timed(lambda i: specv.accept_resample(
        acc_sets[i % ACCEPT_SETS]["target"], acc_sets[i % ACCEPT_SETS]["draft"], acc_sets[i % ACCEPT_SETS]["tokens"],
        parent, T, seed=1234, offset=i, buffers=cbuf), args.steps)
    ms_greedy = timed(lambda i: specv.accept_resample(g_target, None, g_tokens, parent, 0.0, buffers=gbuf),
                      args.steps)
    ms_mask = timed(lambda i: specv.build_tree_mask(parent, out=mask_out), args.steps)
    # the step after verify: KV-cache commit of the accepted paths (a chain's accepted rows are
    # already in place, so this is the validation and bookkeeping cost), on a copy of the cache
    res_c = specv.accept_resample(acc_sets[0]["target"], acc_sets[0]["draft"], acc_sets[0]["tokens"], parent, T,
                                  seed=1234, offset=0)
    kcc, vcc = attn_sets[0][1].clone(), attn_sets[0][2].clone()
    new_ctx = torch.empty_like(ctx_len)
    ms_commit = timed(lambda i: specv.kv_commit(kcc, vcc, ctx_len, res_c.accept_len, res_c.out_nodes, out=new_ctx),
                      args.steps)
    del kcc, vcc

    # measured streaming ceiling on this machine: device-to-device copy of 1 GiB (read + write bytes)
    big = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    big2 = torch.empty_like(big)
    big2.copy_(big)
    ms_copy = timed(lambda i: big2.copy_(big), 5)
    copy_gbs = 2 * (1 << 30) / (ms_copy * 1e-3) / 1e9
    # measured streaming-read ceiling: the library's read probe (the 16-byte non-temporal loads of
    # the streaming kernels) over the same two 1 GiB buffers in turn
    big.fill_(1)
    big2.fill_(2)
    sink = torch.empty(int(specv.lib.specv_read_probe_sink_words()), dtype=torch.int32, device="cuda")
    for i in range(2):
        specv.read_probe(big if i % 2 == 0 else big2, sink)
    ms_read = timed(lambda i: specv.read_probe(big if i % 2 == 0 else big2, sink), 10)
    read_gbs = (1 << 30) / (ms_read * 1e-3) / 1e9
    del big, big2, sink

    acc_sets0_w = acc_sets[0]["w"]
    # acceptance statistics of the timed configuration (set 0)
    res = specv.accept_resample(acc_sets[0]["target"], acc_sets[0]["draft"], acc_sets[0]["tokens"], parent, T,
                                seed=1234, offset=0)
    mean_len = float(res.accept_len.float().mean().item())

    positions = B * K
    n_internal = K
    ab = attn_bytes(CTX, n1)
    cb = accept_bytes(n1, n_internal, V, 2)
    attn_gbs = ab / (ms_attn * 1e-3) / 1e9
    acc_gbs = cb / (ms_accept * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": positions / (ms_step * 1e-3),
        "value_reading": "verify: B*K draft positions / time of one whole step (mask build + tree attention, "
                         "one layer + accept/resample); the accept-only reading is accept_only_positions_per_s",
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "chain verify: B=32, K=5 (6 target positions), V=32000 bf16 logits "
                               "N(0,3), draft noise 0.5285 (alpha~0.8), T=1; attention over ctx 2048 "
                               "(+6 tree keys), 32 q / 8 kv heads, D=128, bf16",
                   "global_batch": B, "seq_len": CTX, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": attn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": attn_gbs / HBM_PEAK_GBS, "traffic": attn_traffic_bytes(),
                     "kernel": "attn_decode_kernel<128,8,1> (specv_tree_attn_verify, one launch)",
                     "bytes_per_call": ab, "ms_per_call": ms_attn,
                     "read_ceiling_gbs": read_gbs, "frac_of_read_ceiling": attn_gbs / read_gbs},
        "roofline_accept": {"bound": "hbm", "achieved": acc_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": acc_gbs / HBM_PEAK_GBS, "traffic": traffic_bytes(ACCEPT_TRAFFIC),
                            "bytes_per_call": cb, "ms_per_call": ms_accept,
                            "kernel": "accept_kernel<bf16> (specv_accept_resample, one launch)",
                            "read_ceiling_gbs": read_gbs, "frac_of_read_ceiling": acc_gbs / read_gbs},
        "accept_only_positions_per_s": positions / (ms_accept * 1e-3),
        "ms_mask": ms_mask,
        "ms_greedy_accept": ms_greedy,
        "ms_kv_commit": ms_commit,
        "mean_accept_len": mean_len,
        "hbm_copy_gbs": copy_gbs,
        "hbm_read_ceiling_gbs": read_gbs,
    }

    del attn_sets, acc_sets
    torch.cuda.empty_cache()
    if not args.no_layer:
        out["verify_layer"] = measure_layer(torch, specv, max(10, args.steps // 4))
    if not args.no_configs:
        # every configuration of the workload list, one after another (inputs resident in HBM)
        out["configs"] = {}
        for name in ("tiny", "chain", "chain-greedy", "eagle", "stress", "ptd"):
            log(f"config {name}")
            out["configs"][name] = measure_config(name, args, torch, specv, workloads)
            for leg in ("accept", "attention"):
                if isinstance(out["configs"][name].get(leg), dict) and "GBps" in out["configs"][name][leg]:
                    out["configs"][name][leg]["frac_of_read_ceiling"] = out["configs"][name][leg]["GBps"] / read_gbs
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(acc_sets0_w, a0)
    print(json.dumps(out))


LAYER_INTER = 14336


def measure_layer(torch, specv, steps):
    """One target layer over the chain step's 192 rows (specv_verify_layer): hidden 4096 (32/8
    heads of 128), MLP width 14336, random-init bf16 weights rotated over two sets (> the
    Infinity Cache), context 2048.  Reports the layer time, the attention call alone on the same
    shape and the weight-streaming rate of the rest (projections + their epilogues)."""
    n1 = K + 1
    hd = HQ * D
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)

    def lin(rows, cols):
        return (torch.randn(rows, cols, generator=gen, device="cuda") / math.sqrt(cols)).to(torch.bfloat16)

    def gain():
        return (1 + 0.2 * torch.randn(hd, generator=gen, device="cuda")).to(torch.bfloat16)

    sets = [specv.LayerWeights(lin((HQ + 2 * HKV) * D, hd), lin(hd, hd), lin(2 * LAYER_INTER, hd),
                               lin(hd, LAYER_INTER), gain(), gain()) for _ in range(2)]
    wbytes = 2 * ((HQ + 2 * HKV) * D * hd + hd * hd + 2 * LAYER_INTER * hd + hd * LAYER_INTER + 2 * hd)
    x = torch.randn(B, n1, hd, generator=gen, device="cuda").to(torch.bfloat16)
    lmax = CTX + n1
    kc = torch.randn(B, HKV, lmax, D, generator=gen, device="cuda").to(torch.bfloat16)
    vc = torch.randn(B, HKV, lmax, D, generator=gen, device="cuda").to(torch.bfloat16)
    ctx = torch.full((B,), CTX, dtype=torch.int32, device="cuda")
    parent = torch.arange(-1, K, dtype=torch.int32, device="cuda").repeat(B, 1)
    mask, depth, _ = specv.build_tree_mask(parent)
    ws = torch.empty((specv.verify_layer_workspace_bytes(B, K, HQ, HKV, D, lmax, LAYER_INTER),), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(x)
    q = torch.randn(B, n1, HQ, D, generator=gen, device="cuda").to(torch.bfloat16)
    abuf = specv.AttnBuffers.allocate(q, kc)

    # the weights also in the tile order the products read (packed once, outside the timed region:
    # a server's weights are static)
    psets = [specv.pack_layer_weights(s_) for s_ in sets]

    def run(i):
        specv.verify_layer(x, psets[i % 2], kc, vc, ctx, mask, depth, HQ, out=out, workspace=ws)

    def run_rowmajor(i):
        specv.verify_layer(x, sets[i % 2], kc, vc, ctx, mask, depth, HQ, out=out, workspace=ws)

    def timed(fn, n):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(n):
            fn(i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n

    for i in range(4):
        run(i)
        run_rowmajor(i)
    ms_layer = timed(run, steps)
    ms_rowmajor = timed(run_rowmajor, steps)
    ms_attn = timed(lambda i: specv.tree_attn_verify(q, kc, vc, ctx, mask, buffers=abuf), steps)
    rest = max(ms_layer - ms_attn, 1e-9)
    gbs = wbytes / (rest * 1e-3) / 1e9
    del sets, psets, kc, vc, ws
    torch.cuda.empty_cache()
    return {"workload": "chain step as one layer: 192 rows, hidden 4096 (32/8 heads of 128), MLP 14336, "
                        "ctx 2048, bf16 random-init weights (packed tile order; ms_rowmajor: row-major)",
            "ms": ms_layer, "ms_rowmajor": ms_rowmajor, "ms_attention_alone": ms_attn,
            "attention_share": ms_attn / ms_layer,
            "weight_bytes": wbytes, "weights_gbs_outside_attention": gbs,
            "weights_hbm_frac_outside_attention": gbs / HBM_PEAK_GBS}


def measure_config(name, args, torch, specv, workloads):
    """Per-kernel times and roofline fractions of one configuration (inputs resident in HBM)."""
    t0 = time.time()
    if name == "tiny":
        w = workloads.tiny_chain_trials(10_000)
        a = workloads.tiny_tree_attention()
    elif name in ("chain", "chain-greedy"):
        w = workloads.chain_config(T=0.0 if name == "chain-greedy" else 1.0)
        a = workloads.chain_attention()
    elif name == "eagle":
        w = workloads.eagle_config()
        a = workloads.eagle_attention(w.parent)
    elif name == "stress":
        w = workloads.stress_config()
        a = workloads.stress_attention()
    else:
        w = workloads.ptd_config()
        a = workloads.ptd_attention(w.parent)
    ldt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    adt = torch.bfloat16 if a.dtype == "bf16" else torch.float32
    tl = torch.from_numpy(np.ascontiguousarray(w.target_logits)).cuda().to(ldt)
    dl = torch.from_numpy(np.ascontiguousarray(w.draft_logits)).cuda().to(ldt) if w.T > 0 else None
    tok = torch.from_numpy(w.tokens).cuda()
    par = torch.from_numpy(w.parent).cuda()
    q = torch.from_numpy(a.q).cuda().to(adt)
    kc = torch.from_numpy(a.k_cache).cuda().to(adt)
    vc = torch.from_numpy(a.v_cache).cuda().to(adt)
    cl = torch.from_numpy(a.ctx_len).cuda()
    apar = torch.from_numpy(a.parent).cuda()
    # a second resident copy (sequences permuted) when one set fits in the 256 MB Infinity Cache
    sets_acc = [(tl, dl, tok, par)]
    acc_bytes = tl.numel() * tl.element_size()
    if acc_bytes < (512 << 20):
        for r in range(1, max(2, int((512 << 20) // max(acc_bytes, 1)) + 1)):
            if r > 24:
                break
            perm = torch.roll(torch.arange(w.B, device="cuda"), r)
            sets_acc.append((tl[perm].contiguous(), None if dl is None else dl[perm].contiguous(), tok[perm].contiguous(),
                             par[perm].contiguous()))
    sets_att = [(q, kc, vc)]
    att_bytes = kc.numel() * kc.element_size() * 2
    if att_bytes < (512 << 20):
        for r in range(1, min(24, int((512 << 20) // att_bytes) + 2)):
            perm = torch.roll(torch.arange(a.q.shape[0], device="cuda"), r)
            sets_att.append((q[perm].contiguous(), kc[perm].contiguous(), vc[perm].contiguous()))
    torch.cuda.synchronize()
    log(f"{name}: inputs ready in {time.time() - t0:.1f} s ({len(sets_acc)} accept sets, {len(sets_att)} attention sets)")

    B, n1 = w.tokens.shape
    V = w.V
    mask_out = specv.build_tree_mask(apar)          # (outputs reused: nothing allocated when timed)
    mask = mask_out[0]
    abuf = specv.AttnBuffers.allocate(q, kc)
    cbuf = specv.AcceptBuffers.allocate(B, n1, V, ldt, "cuda")

    def timed(fn, n):
        for i in range(3):
            fn(i)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(n):
            fn(i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n

    steps = max(20, min(args.steps, 200))
    ms_mask = timed(lambda i: specv.build_tree_mask(apar, out=mask_out), steps)
    ms_attn = timed(lambda i: specv.tree_attn_verify(*sets_att[i % len(sets_att)], cl, mask, a.scale, buffers=abuf),
                    steps)
    ms_acc = timed(lambda i: specv.accept_resample(*sets_acc[i % len(sets_acc)], w.T, seed=1, offset=i,
                                                   buffers=cbuf), steps)
    # one level of draft-tree construction at this configuration's vocabulary: 16 frontier rows
    # per sequence, k = 3 (EAGLE) or 4 (the PTD width cap), 16 kept; rotated sets of resident rows
    expand_info = None
    elem = 2 if w.dtype == "bf16" else 4
    if name in ("eagle", "ptd"):
        kx, FX = (3 if name == "eagle" else 4), 16
        row_bytes = B * FX * V * elem
        nsets = max(1, min(8, int((512 << 20) // row_bytes) + 1))
        gen = torch.Generator(device="cuda")
        gen.manual_seed(11)
        xsets = [(torch.randn((B, FX, V), generator=gen, device="cuda") * 3.0).to(ldt) for _ in range(nsets)]
        xtree = specv.DraftTree.with_roots(torch.zeros(B, dtype=torch.int32, device="cuda"), 1024)
        xtree.n_nodes.fill_(1 + FX)
        xfront = torch.arange(1, FX + 1, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
        xout = torch.empty((B, FX), dtype=torch.int32, device="cuda")
        xws = torch.empty((specv.tree_expand_workspace_bytes(B, FX),), dtype=torch.uint8, device="cuda")
        ms_x = timed(lambda i: specv.tree_expand(xsets[i % nsets], xfront, xtree, kx, w.T, FX, new_frontier=xout,
                                                 workspace=xws), steps)
        expand_info = {"ms": ms_x, "frontier_rows": B * FX, "k": kx, "bytes": row_bytes,
                       "GBps": row_bytes / (ms_x * 1e-3) / 1e9,
                       "hbm_frac": row_bytes / (ms_x * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del xsets

    # the accept rule for the other sibling draftings, same inputs (the time does not depend on how
    # the tokens were drafted beyond the walk's path; fixed candidates read no draft rows)
    ms_acc_rule = {}
    if n1 > 2 and w.T > 0:
        for rule in ("iid", "deterministic"):
            ms_acc_rule[rule] = timed(lambda i: specv.accept_resample(
                sets_acc[i % len(sets_acc)][0], None if rule == "deterministic" else sets_acc[i % len(sets_acc)][1],
                *sets_acc[i % len(sets_acc)][2:], w.T, seed=1, offset=i, buffers=cbuf, siblings=rule), steps)
    r = specv.accept_resample(tl, dl, tok, par, w.T, seed=1, offset=0, buffers=cbuf)
    accept_len = r.accept_len.cpu().numpy()
    out_nodes = r.out_nodes.cpu().numpy()
    # KV-cache commit of the accepted paths (the step after the verify step, not part of it), on a
    # copy of the cache; every call moves the same rows
    # (the tiny case's accept trials and its attention tree are different batches: no commit leg)
    ms_commit, moved = None, 0
    if (B, n1) == tuple(a.parent.shape):
        kcc, vcc = kc.clone(), vc.clone()
        new_ctx = torch.empty_like(cl)
        ms_commit = timed(lambda i: specv.kv_commit(kcc, vcc, cl, r.accept_len, r.out_nodes, out=new_ctx), steps)
        moved = sum(1 for b in range(B) for d in range(1, int(accept_len[b]) + 1) if out_nodes[b, d - 1] != d)
        del kcc, vcc

    # algorithmic work
    pa = w.parent
    internal = sum(len(set(int(x) for x in pa[b, 1:])) for b in range(B))
    elem = 2 if w.dtype == "bf16" else 4
    acc_b = (B * n1 + (internal if w.T > 0 else 0)) * V * elem
    Bq, _, Hq, D = a.q.shape
    Hkv = a.k_cache.shape[1]
    esz = 2 if a.dtype == "bf16" else 4
    keys = int(a.ctx_len.sum()) + Bq * n1
    att_b = 2 * Hkv * keys * D * esz + 2 * Bq * n1 * Hq * D * esz
    att_f = 4.0 * Hq * D * sum(int(a.ctx_len[b]) + n1 for b in range(Bq)) * n1
    positions = B * (n1 - 1)
    out = {
        "config": name, "description": CONFIGS[name], "B": B, "nodes": n1, "V": V, "T": w.T,
        "internal_nodes": internal,
        "ms_mask": ms_mask, "ms_attention": ms_attn, "ms_accept": ms_acc,
        "attention": {"bytes": att_b, "flops": att_f, "GBps": att_b / (ms_attn * 1e-3) / 1e9,
                      "hbm_frac": att_b / (ms_attn * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "TFLOPs": att_f / (ms_attn * 1e-3) / 1e12,
                      "mfma_frac": att_f / (ms_attn * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS,
                      "arith_intensity": att_f / att_b},
        "accept": {"bytes": acc_b, "GBps": acc_b / (ms_acc * 1e-3) / 1e9,
                   "hbm_frac": acc_b / (ms_acc * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "accept_other_sibling_rules": {rule: {"ms": ms, "bytes": (B * n1 + (internal if rule == "iid" else 0)) * V * elem,
                                              "hbm_frac": (B * n1 + (internal if rule == "iid" else 0)) * V * elem
                                              / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
                                       for rule, ms in ms_acc_rule.items()},
        "tree_expand": expand_info,
        "kv_commit": {"ms": ms_commit, "rows_moved": moved,
                      "bytes": moved * 2 * 2 * a.k_cache.shape[1] * a.q.shape[3] * (2 if a.dtype == "bf16" else 4)},
        "positions_per_s_accept_only": positions / (ms_acc * 1e-3),
        "positions_per_s_verify": positions / ((ms_mask + ms_attn + ms_acc) * 1e-3),
        "mean_tokens_per_step": float(np.mean(accept_len + 1)),
        "acceptance": acceptance_stats(torch, w, tl, dl, accept_len),
    }
    del sets_acc, sets_att, tl, dl, q, kc, vc
    torch.cuda.empty_cache()
    return out


def acceptance_stats(torch, w, tl, dl, accept_len):
    """Per-position acceptance rate alpha = sum_x min(p(x), q(x)) (the lesson, "Expected Speedup";
    the review, section 2 "Efficiency analysis") from the logits of the draft nodes' parent rows,
    and, for chains, the expected tokens per step (1 - alpha^(K+1)) / (1 - alpha) beside the
    measured mean of accept_len + 1.  Computed here with torch (a measurement, not the verify
    path)."""
    B, n1 = w.tokens.shape
    out = {"mean_tokens_measured": float(np.mean(accept_len + 1))}
    if w.T <= 0 or dl is None or n1 < 2:
        out["note"] = "greedy or no draft positions: alpha not defined by the sampling rule"
        return out
    chain = bool(np.all(w.parent[:, 1:] == np.arange(n1 - 1)[None, :]))

    def alpha_rows(t_rows, d_rows):
        pt = torch.softmax(t_rows.float() / w.T, dim=-1)
        qt = torch.softmax(d_rows.float() / w.T, dim=-1)
        return torch.minimum(pt, qt).sum(dim=-1).double().cpu().numpy().ravel()

    if chain:
        a = np.concatenate([alpha_rows(tl[b0:b0 + 256, :n1 - 1], dl[b0:b0 + 256, :n1 - 1])
                            for b0 in range(0, B, 256)])
    else:
        a = np.concatenate([alpha_rows(tl[b, sorted(set(int(x) for x in w.parent[b, 1:]))],
                                       dl[b, sorted(set(int(x) for x in w.parent[b, 1:]))]) for b in range(B)])
    out["alpha_mean"] = float(a.mean())
    out["alpha_min"] = float(a.min())
    out["alpha_max"] = float(a.max())
    if chain:
        K = n1 - 1
        al = float(a.mean())
        out["expected_tokens_closed_form"] = (1.0 - al ** (K + 1)) / (1.0 - al) if al < 1 else float(K + 1)
        out["closed_form"] = "(1 - alpha^(K+1)) / (1 - alpha), alpha = mean over positions"
        # the same expectation with each position's own alpha (the draft tokens here are drawn
        # independently per position, so acceptances are independent Bernoulli(alpha_j)):
        # E = sum_k prod_{j<k} alpha_j, averaged over the sequences
        ab = a.reshape(B, K)
        out["expected_tokens_per_position_alpha"] = float(np.mean(
            1.0 + np.sum(np.cumprod(ab, axis=1), axis=1)))
        sd = float(np.std(accept_len + 1))
        out["measured_std_error"] = sd / math.sqrt(B)
    else:
        out["note"] = "tree: alpha over the internal nodes' rows; the chain closed form does not apply"
    return out


def cpu_baseline(w, a):
    """Oracle (numpy fp64) on a bounded sample of the same workload: the whole verify step
    (mask, attention, accept) for as many sequences as fit in about 15 s on all the host threads
    numpy uses, then about 5 s on one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import accept as o_accept, attention as o_attn, philox as o_philox, tree as o_tree

    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])

    def run(seconds):
        t0 = time.time()
        done = 0
        while time.time() - t0 < seconds:
            b = done % w.B
            mask, _, _ = o_tree.build_tree_mask_batch(a.parent[b:b + 1])
            o_attn.tree_attention(a.q[b:b + 1], a.k_cache[b:b + 1], a.v_cache[b:b + 1], a.ctx_len[b:b + 1], mask,
                                  a.scale)
            ua, ur = o_philox.uniforms(1234, 0, 1, w.N1)
            o_accept.accept_batch(np.asarray(w.target_logits[b:b + 1], np.float64),
                                  np.asarray(w.draft_logits[b:b + 1], np.float64),
                                  w.tokens[b:b + 1], w.parent[b:b + 1], w.T, ua, ur)
            done += 1
        return done, time.time() - t0

    done, dt = run(15.0)
    with threadpool_limits(limits=1):
        done1, dt1 = run(5.0)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": done * K / dt, "unit": "positions/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} sequences (cycling over the {w.B} of the timed workload), whole verify "
                      f"step (mask, attention, accept) in numpy fp64, {dt:.1f} s",
            "value_one_thread": done1 * K / dt1, "cpu_model": model}


if __name__ == "__main__":
    main()
