"""Benchmark of the compressed-key indexer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only] [--no-cpu-baseline]
                    [--only NAME] [--copy-calibration]

--only NAME runs one secondary workload alone and prints its line (for profiler runs of one
kernel); --copy-calibration runs plain 1 GiB device copies (the reference for scaling the
profiler's FETCH_SIZE / WRITE_SIZE counters).

Headline step: decode scoring of 32 requests x 65,536 bf16 compressed entries (256K-token
context at 4:1 compression, 1,024 pages of 64 per request, pages scattered by a permuted block
table, 10% planted hot pages) with their top-512, in one fm_index_topk call (scoring and
selection fused); the two-call path (fm_index_logits, then fm_topk512) is timed beside it.
The pool is replicated on the device and the replicas rotate from step to step
so that no step finds its keys in the 256 MB Infinity Cache.  The metric is compressed entries
scored and selected per second over the whole call; every input is resident in HBM before the
timed region starts.

The timed steps are those calls captured into HIP graphs and replayed (the pages run this step
inside a CUDA graph): one graph holds three consecutive steps, one call per pool replica, as a
model's decode graph holds one indexer call per layer, so host launch latency and the per-graph
launch cost stay out of the step; the eager rate of the same calls is reported beside it.
Per-kernel durations come from HIP events recorded on the stream the kernels run on.  The
roofline object reports the fused call against HBM peak (8 TB/s) with its algorithmic bytes
(keys once, q/w once, block table, indices written) over its average duration: HIP events
around the same calls launched back to back (events around each single call, which add a
few microseconds, are reported beside it as bracketed_ms).  Secondary entries measure the other
workloads (one call a step, timed over the calls back to back): the three-layer fp8 mask with
64 heads, with one pool shared by the three encoders, and with the retriever's 128 heads,
two-level fp8 scoring over 384 resident pages, causal fp8 prefill, Mode A end to end (the
three-encoder mask, then the masked top-512 of 21 layers x 8 requests over 262,144 entries,
every layer scoring its own fp8 pool), the retriever's query encoder at
decode and prefill batch sizes, and golden-label construction from 128 tokens x 21 layers x
65,536 selector scores.  Beside the published peaks, the line carries measured ceilings: a
plain 1 GiB device copy (HBM) and the vendor GEMM library's fp8 and bf16 rates on random
8192^3 products (dense MFMA); the MFMA-bound secondaries report their fraction of the latter.
cpu_baseline times the fp64 oracle on a bounded sample of the headline workload on the host
cores.

Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CPU_BASELINES = True         # oracle timings beside each secondary line (off: --no-cpu-baseline)
FP8_PEAK_TFLOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0
FLOP_PER_PAIR = 2 * 64 * 128


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "top_selection_fm_amd", "csrc"))):
        with open(os.path.join(ROOT, "top_selection_fm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(name: str, digest: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was taken on
    the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources") != digest:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events on the current (launch) stream.  With several names, events around each
    call of each step (per-call brackets); with one name, one event before the first call and
    one after the last, so the average covers the calls back to back (brackets around every
    single call add a few microseconds of their own)."""

    def __init__(self, torch, names, steps):
        self.torch = torch
        self.names = names
        self.steps = steps
        self.b2b = len(names) == 1
        n_ev = 1 if self.b2b else steps
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
                   for _ in range(n_ev)]

    def mark(self, step, i):
        if not self.b2b:
            self.ev[step][i].record()
        elif (step == 0 and i == 0) or (step == self.steps - 1 and i == 1):
            self.ev[0][i].record()

    def per_kernel_ms(self):
        if self.b2b:
            return {self.names[0]: self.ev[0][0].elapsed_time(self.ev[0][1]) / self.steps}
        out = {}
        for i, n in enumerate(self.names):
            out[n] = float(np.mean([e[i].elapsed_time(e[i + 1]) for e in self.ev]))
        return out


def timed(torch, names, fn, steps, warmup):
    for s in range(warmup):
        fn(s, None)
    torch.cuda.synchronize()
    tm = Timer(torch, names, steps)
    t0 = time.perf_counter()
    for s in range(steps):
        fn(s, tm)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, tm.per_kernel_ms()


# ----------------------------------------------------------------------------- workloads
def graph_time(torch, calls, steps, warmup):
    """`calls` (one step each, one per pool replica) captured in order into one HIP graph, as a
    model's decode graph holds one indexer call per layer, and replayed; steps left over when
    `steps` is not a multiple of len(calls) replay single-call graphs.  Steps s = 0, 1, ...
    run calls[s % len(calls)] in turn either way.  Returns (wall seconds, event ms per step)."""
    n = len(calls)
    whole = torch.cuda.CUDAGraph()
    with torch.cuda.graph(whole):
        for c in calls:
            c()
    single = []
    for c in calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            c()
        single.append(g)

    def run(k):
        for _ in range(k // n):
            whole.replay()
        for s in range(k % n):
            single[s].replay()

    run(warmup)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    g0.record()
    run(steps)
    g1.record()
    torch.cuda.synchronize()
    return time.perf_counter() - t0, g0.elapsed_time(g1) / steps


def b2b_ms(torch, call, steps, warmup):
    """Average duration of `call(step)` launched back to back, between two events on the
    launch stream (events around every single call would add their own few us)."""
    for s in range(warmup):
        call(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(steps):
        call(s)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def run_decode(torch, api, W, steps, warmup, replicas=3):
    """The decode step: one fm_index_topk call (scoring and top-512 fused) over 32 requests x
    65,536 bf16 entries; the two-call path (fm_index_logits + fm_topk512) is timed beside it."""
    wl = W.decode_bf16()
    dw = api.DeviceWorkload(wl, "cuda:0", pool_copies=replicas)
    B = wl.kv.B
    ld = wl.kv.block_table.shape[1] * 64
    idx = torch.empty((B, 512), dtype=torch.int32, device="cuda:0")
    nb = api.fm_workspace_bytes(api.FM_OP_INDEX_TOPK, B, ld)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    q = dw.query()
    kvs = [dw.kv(r) for r in range(replicas)]

    def fused(s):
        api.fm_index_topk(q, kvs[s % replicas], None, 0, 512, idx, None, None, 0, ws, nb)

    def step(s, tm):
        if tm: tm.mark(s, 0)
        fused(s)
        if tm: tm.mark(s, 1)

    wall, per = timed(torch, ["index_topk"], step, steps, warmup)
    graph_wall, graph_ms = graph_time(torch, [lambda r=r: fused(r) for r in range(replicas)],
                                      steps, warmup)
    fused_ms = b2b_ms(torch, fused, steps, warmup)
    # the two-call path: logits to memory, then the top-k kernel
    logits = torch.empty((B, ld), dtype=torch.float32, device="cuda:0")
    nbt = api.fm_workspace_bytes(api.FM_OP_TOPK, B, ld)
    wst = torch.empty(max(nbt, 16), dtype=torch.uint8, device="cuda:0")

    def two(s):
        api.fm_index_logits(q, kvs[s % replicas], logits, ld)
        api.fm_topk512(logits, ld, B, None, None, 0, None, 512, idx, None, wst, nbt)

    two_wall, two_graph_ms = graph_time(torch, [lambda r=r: two(r) for r in range(replicas)],
                                        steps, warmup)
    score_ms = b2b_ms(torch, lambda s: api.fm_index_logits(q, kvs[s % replicas], logits, ld),
                      steps, warmup)
    entries = int(wl.kv.seq_lens.sum())
    key_bytes = entries * 256
    alg_bytes = key_bytes + B * 64 * 128 * 2 + B * 64 * 2 + wl.kv.block_table.nbytes + \
        wl.kv.seq_lens.nbytes + B * 512 * 4
    return wl, dict(entries=entries, wall_s=wall, per=per, alg_bytes=alg_bytes,
                    flops=entries * FLOP_PER_PAIR, graph_wall_s=graph_wall, graph_ms=graph_ms,
                    fused_b2b_ms=fused_ms, two_call=dict(
                        ms_per_step=two_wall / steps * 1e3, graph_event_ms=two_graph_ms,
                        score_kernel_ms=score_ms,
                        score_hbm_frac=(alg_bytes + B * ld * 4 - B * 512 * 4) / (score_ms * 1e-3)
                        / 1e9 / HBM_PEAK_GBS))


def run_mask(torch, api, W, steps, warmup, replicas=2, heads=64, shared=False):
    """Level-1 mask of three encoders over 8 x 262,144 fp8 entries.  shared: the three
    encoders score one pool (passed three times), so each key is read once for all of them
    and the call is bounded by bf16 MFMA rather than HBM."""
    wl = W.three_layer_mask_fp8(heads=heads, shared_keys=shared)
    dw = api.DeviceWorkload(wl, "cuda:0", pool_copies=replicas)
    B = wl.kv.B
    ld = wl.kv.block_table.shape[1] * 64
    n_pages = ld // 64
    mask = torch.empty((B, ld), dtype=torch.uint8, device="cuda:0")
    cnt = torch.empty(B, dtype=torch.int32, device="cuda:0")
    plist = torch.empty((B, n_pages), dtype=torch.int32, device="cuda:0")
    qs = [dw.query(l) for l in range(3)]
    if shared:
        kvs = [api.kv_desc([dw.replicas[r][0]] * 3, "fp8x132", dw.block_table, dw.seq_lens,
                           dw.max_seq_len) for r in range(replicas)]
    else:
        kvs = [dw.kv(r) for r in range(replicas)]

    def step(s, tm):
        if tm: tm.mark(s, 0)
        api.fm_resident_mask(qs, kvs[s % replicas], api.FM_UNION_MAX, 0.5, 0, 0, mask, ld, cnt,
                             plist, n_pages)
        if tm: tm.mark(s, 1)

    wall, per = timed(torch, ["mask+compact"], step, steps, warmup)
    ms = b2b_ms(torch, lambda s: step(s, None), steps, warmup)
    entries = int(wl.kv.seq_lens.sum())
    cpu = None
    if CPU_BASELINES and heads == 64 and not shared:
        import oracle
        dt, cores, _ = cpu_time(lambda: oracle.resident_mask(wl))
        cpu = dict(value=entries / dt, unit="entries/s", cores=cores, kind="oracle",
                   sample=f"whole workload (3 encoders x {entries} entries, fp64), {dt:.1f} s")
    alg = (1 if shared else 3) * entries * 132 + 3 * B * (heads * 128 * 2 + heads * 2) + \
        wl.kv.block_table.nbytes + B * ld + B * n_pages * 4
    flops = 3 * entries * 2 * heads * 128
    sec = ms * 1e-3
    return dict(workload=wl.name + ("" if heads == 64 else f"_h{heads}") +
                ("_shared_keys" if shared else ""), entries=entries,
                bound="bf16 mfma" if shared else "hbm",
                layers=3, heads=heads, ms=ms, bracketed_ms=per["mask+compact"],
                entries_per_s=entries / sec,
                hbm_gbs=alg / sec / 1e9, hbm_frac=alg / sec / 1e9 / HBM_PEAK_GBS,
                alg_bytes=alg, mfma_tflops=flops / sec / 1e12,
                bf16_mfma_frac=flops / sec / 1e12 / BF16_PEAK_TFLOPS, cpu_baseline=cpu)


def run_two_level(torch, api, W, steps, warmup, replicas=12):
    wl = W.two_level_resident_fp8()
    dw = api.DeviceWorkload(wl, "cuda:0", pool_copies=replicas)
    T = wl.queries[0].T
    res_ld = wl.resident_pages.shape[1]
    nb = api.fm_workspace_bytes(api.FM_OP_SCORE_RESIDENT, T, res_ld * 64)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    idx = torch.empty((T, 512), dtype=torch.int32, device="cuda:0")
    q = dw.query()
    kvs = [dw.kv(r) for r in range(replicas)]

    def step(s, tm):
        if tm: tm.mark(s, 0)
        api.fm_score_resident(q, kvs[s % replicas], dw.resident_pages, dw.n_resident, res_ld,
                              512, idx, None, ws, nb)
        if tm: tm.mark(s, 1)

    wall, per = timed(torch, ["score_resident"], step, steps, warmup)
    ms = b2b_ms(torch, lambda s: step(s, None), steps, warmup)
    entries = int(wl.n_resident.sum()) * 64
    cpu = None
    if CPU_BASELINES:
        import oracle
        dt, cores, _ = cpu_time(lambda: oracle.score_resident(wl))
        cpu = dict(value=entries / dt, unit="entries/s", cores=cores, kind="oracle",
                   sample=f"whole workload ({entries} resident entries, fp64 + top-512), "
                          f"{dt:.2f} s")
    alg = entries * 132 + T * (64 * 128 * 2 + 64 * 2) + wl.resident_pages.nbytes + \
        int(wl.n_resident.sum()) * 4 + T * 512 * 4
    return dict(workload=wl.name, entries=entries, ms=ms, bracketed_ms=per["score_resident"],
                entries_per_s=entries / (ms * 1e-3),
                hbm_gbs=alg / (ms * 1e-3) / 1e9, hbm_frac=alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                alg_bytes=alg, note="score + top-512 in one call (two kernels)", cpu_baseline=cpu)


def run_prefill(torch, api, W, steps, warmup):
    wl = W.prefill_causal_fp8()
    dw = api.DeviceWorkload(wl, "cuda:0")
    T = wl.queries[0].T
    ld = wl.kv.max_seq_len
    logits = torch.empty((T, ld), dtype=torch.float32, device="cuda:0")
    idx = torch.empty((T, 512), dtype=torch.int32, device="cuda:0")
    nb = api.fm_workspace_bytes(api.FM_OP_TOPK, T, ld)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    q, kv = dw.query(), dw.kv()
    # each row's visible length (its causal cut): the top-k reads no further
    n_vis = np.minimum(wl.queries[0].q_pos.astype(np.int64) // 4, ld).astype(np.int32)
    n_valid = torch.from_numpy(n_vis).to("cuda:0")

    def step(s, tm):
        if tm: tm.mark(s, 0)
        api.fm_index_logits(q, kv, logits, ld)
        if tm: tm.mark(s, 1)
        api.fm_topk512(logits, ld, T, n_valid, None, 0, None, 512, idx, None, ws, nb)
        if tm: tm.mark(s, 2)

    wall, per = timed(torch, ["score", "topk"], step, steps, warmup)
    score_ms = b2b_ms(torch, lambda s: api.fm_index_logits(q, kv, logits, ld), steps, warmup)
    topk_ms = b2b_ms(torch, lambda s: api.fm_topk512(logits, ld, T, n_valid, None, 0, None, 512,
                                                      idx, None, ws, nb), steps, warmup)
    pairs = int(sum(min(ld, p // 4) for p in wl.queries[0].q_pos.tolist()))
    cpu = None
    if CPU_BASELINES:
        import oracle
        rows = np.arange(0, T, 16, dtype=np.int32)          # every 16th row: 1/16 of the pairs
        sub = int(sum(min(ld, int(wl.queries[0].q_pos[r]) // 4) for r in rows))

        def run():
            oracle.topk_rows(oracle.logits(wl, rows=rows))

        dt, cores, _ = cpu_time(run)
        cpu = dict(value=sub / dt, unit="pairs/s", cores=cores, kind="oracle",
                   sample=f"{rows.size} of {T} rows (every 16th; {sub} of {pairs} visible "
                          f"pairs, fp64 logits + top-512) in {dt:.1f} s; whole workload "
                          f"scaled linearly: {dt * pairs / sub:.0f} s")
    flops = pairs * FLOP_PER_PAIR
    return dict(workload=wl.name, visible_pairs=pairs, score_ms=score_ms, topk_ms=topk_ms,
                bracketed_ms=per, pairs_per_s=pairs / ((score_ms + topk_ms) * 1e-3),
                mfma_tflops=flops / (score_ms * 1e-3) / 1e12,
                mfma_frac=flops / (score_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS,
                cpu_baseline=cpu)


def run_mode_a(torch, api, W, steps, warmup):
    """Mode A end to end over 8 requests x 262,144 entries: the Level-1 mask of three fp8
    encoders (fm_resident_mask), then one fm_index_topk call over the 21 layers x 8 requests
    rows, each layer scoring its own fp8 pool (row_pool) under its request's mask (row_req).
    The scoring alone (fm_index_logits over the same rows) is timed beside it, so the
    selection's share is level2 - scoring."""
    wl = W.mode_a_fp8()
    dw = api.DeviceWorkload(wl, "cuda:0")
    B, n_enc = wl.kv.B, 3
    q2w = wl.queries[n_enc]
    T = q2w.T
    ld = wl.kv.block_table.shape[1] * 64
    n_pages = ld // 64
    dev = "cuda:0"
    mask = torch.empty((B, ld), dtype=torch.uint8, device=dev)
    cnt = torch.empty(B, dtype=torch.int32, device=dev)
    dens = torch.empty((B, n_pages), dtype=torch.int32, device=dev)
    idx = torch.empty((T, 512), dtype=torch.int32, device=dev)
    nb = api.fm_workspace_bytes(api.FM_OP_INDEX_TOPK, T, ld)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    q_enc = [dw.query(l) for l in range(n_enc)]
    kv_enc, kv_all = dw.kv(0, list(range(n_enc))), dw.kv()
    q2 = dw.query(n_enc)

    def level1(s):
        api.fm_resident_mask(q_enc, kv_enc, api.FM_UNION_MAX, 0.5, 0, 0, mask, ld, cnt, None, 0,
                             dens)

    def level2(s):
        api.fm_index_topk(q2, kv_all, mask, ld, 512, idx, None, None, 0, ws, nb)

    def step(s, tm):
        if tm: tm.mark(s, 0)
        level1(s)
        if tm: tm.mark(s, 1)
        level2(s)
        if tm: tm.mark(s, 2)

    wall, per = timed(torch, ["level1", "level2"], step, steps, warmup)
    l1_ms = b2b_ms(torch, level1, steps, warmup)
    l2_ms = b2b_ms(torch, level2, steps, warmup)
    del ws
    logits = torch.empty((T, ld), dtype=torch.float32, device=dev)
    score_ms = b2b_ms(torch, lambda s: api.fm_index_logits(q2, kv_all, logits, ld), steps, warmup)
    del logits
    n_vis = int(wl.kv.seq_lens.sum())     # one layer over all requests (a row sees its own)
    resident = int(mask.sum().item())
    l1_alg = n_enc * n_vis * 132 + n_enc * B * (64 * 128 * 2 + 64 * 2) + \
        wl.kv.block_table.nbytes + B * ld + B * n_pages * 4
    # Level 2: every layer's keys once, queries and weights, the block table and the mask once
    # per row, the output
    l2_alg = (T // B) * n_vis * 132 + T * (64 * 128 * 2 + 64 * 2) + (T // B) * (
        wl.kv.block_table.nbytes + B * ld) + T * 512 * 4
    step_ms = wall / steps * 1e3
    return dict(workload=f"mode_a_fp8_b{B}_l{T // B}_s{ld}_top512", rows=T,
                candidates=(T // B) * n_vis, resident_entries_per_request=resident / B,
                ms_per_step=step_ms, entries_per_s=(T // B) * n_vis / (step_ms * 1e-3),
                level1_ms=l1_ms, level2_ms=l2_ms, level2_scoring_only_ms=score_ms,
                level2_selection_share=max(0.0, 1 - score_ms / l2_ms),
                level1_share=l1_ms / (l1_ms + l2_ms),
                bracketed_ms=per,
                level1_hbm_frac=l1_alg / (l1_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                level2_hbm_frac=l2_alg / (l2_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                alg_bytes=dict(level1=l1_alg, level2=l2_alg),
                note="Level-1 mask (3 encoders) + masked top-512 of 21 layers, each over "
                     "its own fp8 pool, in one call")


def run_labels(torch, api, W, steps, warmup):
    """Golden labels for retriever training: 128 future tokens x 21 CSA layers x 65,536
    compressed entries (256K context at 4:1) of synthetic selector scores, nucleus p = 0.6,
    3 votes, lookahead tau = 64 (65 windows).  The pass reads every score once."""
    g = W.selector_scores()
    dev = "cuda:0"
    S = torch.from_numpy(g.scores).to(dev)
    nv = torch.from_numpy(g.n_valid).to(dev)
    T, L, ld, tau = g.T, g.n_layers, g.ld, 64
    nb = api.fm_golden_workspace_bytes(T, L, ld, tau)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    ptr = torch.empty(T - tau + 2, dtype=torch.int32, device=dev)
    cap = (T - tau + 1) * 4096
    idx = torch.empty(cap, dtype=torch.int32, device=dev)
    sc = torch.empty(cap, dtype=torch.float32, device=dev)

    def step(s, tm):
        if tm: tm.mark(s, 0)
        api.fm_golden_labels(S, ld, T, L, nv, 0.6, 3, tau, ptr, idx, sc, cap, ws, nb)
        if tm: tm.mark(s, 1)

    wall, per = timed(torch, ["labels"], step, steps, warmup)
    ms = b2b_ms(torch, lambda s: step(s, None), steps, warmup)
    n_labels = int(ptr[-1].item())
    alg = S.numel() * 4 + nv.numel() * 4 + ptr.numel() * 4 + n_labels * 8
    return dict(workload=g.name + f"_tau{tau}", rows=T * L, scores=S.numel(), ms=ms,
                bracketed_ms=per["labels"],
                scores_per_s=S.numel() / (ms * 1e-3), hbm_gbs=alg / (ms * 1e-3) / 1e9,
                hbm_frac=alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, alg_bytes=alg,
                labels=n_labels, windows=T - tau + 1)


def run_encoder(torch, api, W, steps, warmup):
    """The retriever's query encoder at the page's sizes (d_model 4096, q_rank 2048, 128 heads
    of 128, RoPE on 64 dims): a decode batch of 32 rows (weight-bandwidth bound) and a prefill
    batch of 4,096 rows (bf16 MFMA bound), synthetic weights and hidden states."""
    out = {}
    for T in (32, 4096):
        e = W.query_encoder(T=T)
        dev = "cuda:0"
        t = {k: torch.from_numpy(getattr(e, k).view(np.int16)).to(dev)
             for k in ("hidden", "wq_a", "q_norm", "wq_b", "w_proj")}
        pos = torch.from_numpy(e.pos).to(dev)
        desc = api.encoder_desc(t["wq_a"], t["q_norm"], t["wq_b"], t["w_proj"],
                                n_heads=e.n_heads, d_model=e.d_model, q_rank=e.q_rank)
        nb = api.fm_encode_workspace_bytes(desc, T)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        q = torch.empty((T, e.n_heads, 128), dtype=torch.bfloat16, device=dev)
        w = torch.empty((T, e.n_heads), dtype=torch.float32, device=dev)

        def step(s, tm):
            if tm: tm.mark(s, 0)
            api.fm_encode_queries(desc, t["hidden"], T, pos, q, w, ws, nb)
            if tm: tm.mark(s, 1)

        wall, per = timed(torch, ["encode"], step, steps, warmup)
        ms = b2b_ms(torch, lambda s: step(s, None), steps, warmup)
        wbytes = sum(t[k].numel() * 2 for k in ("wq_a", "q_norm", "wq_b", "w_proj"))
        alg = wbytes + t["hidden"].numel() * 2 + T * 4 + q.numel() * 2 + w.numel() * 4
        flops = 2 * T * (e.d_model * (e.q_rank + e.n_heads) + e.q_rank * e.n_heads * 128)
        out[f"t{T}"] = dict(rows=T, ms=ms, bracketed_ms=per["encode"],
                            rows_per_s=T / (ms * 1e-3),
                            hbm_gbs=alg / (ms * 1e-3) / 1e9,
                            hbm_frac=alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                            mfma_tflops=flops / (ms * 1e-3) / 1e12,
                            mfma_frac=flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                            alg_bytes=alg, flops=flops)
        del t, ws, q, w
    return dict(workload="query_encoder_d4096_r2048_h128", **out)


# ----------------------------------------------------------------------------- CPU baseline
def cpu_baseline(wl, budget_s=12.0):
    import oracle

    oracle.lib()
    done_entries = 0
    t0 = time.perf_counter()
    rows = 0
    for b in range(wl.kv.B):
        L = oracle.logits(wl, rows=[b])
        oracle.topk_rows(L)
        done_entries += int(wl.kv.seq_lens[b])
        rows += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=done_entries / dt, unit="entries/s", cores=oracle.num_threads(),
                kind="oracle",
                sample=f"{rows} of {wl.kv.B} requests of the headline workload "
                       f"({done_entries} entries, fp64 logits + top-512), {dt:.1f} s")


def cpu_c1_single_thread(W, budget_s=1.0):
    """The 4,096-entry fp32 single-query workload: fp64 logits + top-512 on one thread."""
    import oracle

    wl = W.tiny_single_query()
    n0 = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.topk_rows(oracle.logits(wl))
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(n0)
    n = int(wl.kv.seq_lens.sum())
    return dict(value=n * reps / dt, unit="entries/s", cores=1, kind="oracle",
                sample=f"{reps} passes over the whole workload ({n} entries), {dt:.2f} s",
                ms_per_pass=dt / reps * 1e3)


def cpu_time(fn):
    import oracle

    oracle.lib()
    t0 = time.perf_counter()
    out = fn()
    return time.perf_counter() - t0, oracle.num_threads(), out


def copy_calibration(torch, nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").random_(0, 255)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {nbytes} bytes")


def vendor_gemm_tflops(torch, n=8192, reps=20):
    """Measured dense-MFMA ceilings on this GPU: the vendor GEMM library (through torch) on
    n x n x n products of random operands, fp8 E4M3 (scaled, bf16 output) and bf16.  Random
    operands matter: the chip's clock drops under their power, so zero or constant operands
    would overstate the ceiling.  None where the library offers no kernel."""
    def rate(fn):
        for _ in range(3):
            fn()
        ms = b2b_ms(torch, lambda s: fn(), reps, 0)
        return 2.0 * n * n * n / (ms * 1e-3) / 1e12
    out = {}
    g = torch.Generator(device="cuda:0").manual_seed(7)
    a = torch.randn(n, n, device="cuda:0", generator=g) * 0.5
    b = torch.randn(n, n, device="cuda:0", generator=g) * 0.5
    try:
        a8, b8 = a.to(torch.float8_e4m3fn), b.to(torch.float8_e4m3fn).t()
        one = torch.tensor(1.0, device="cuda:0")
        out["fp8_gemm_tflops"] = rate(lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one,
                                                               out_dtype=torch.bfloat16))
        del a8, b8
    except Exception as e:  # torch without an fp8 GEMM: report the gap, keep the rest
        out["fp8_gemm_tflops"] = None
        log(f"fp8 GEMM ceiling unavailable: {e!r}")
    try:
        ab, bb = a.to(torch.bfloat16), b.to(torch.bfloat16)
        out["bf16_gemm_tflops"] = rate(lambda: ab @ bb)
        del ab, bb
    except Exception as e:
        out["bf16_gemm_tflops"] = None
        log(f"bf16 GEMM ceiling unavailable: {e!r}")
    out["how"] = f"vendor GEMM {n}^3, random operands, events around {reps} back-to-back calls"
    del a, b
    torch.cuda.empty_cache()
    return out


def stream_copy_gbs(torch, nbytes=1 << 30, reps=10):
    """Measured HBM rate of a plain 1 GiB device-to-device copy (bytes read + written)."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").random_(0, 255)
    b = torch.empty_like(a)
    ms = b2b_ms(torch, lambda s: b.copy_(a), reps, 2)
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--only", default=None)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the "
              f"indexer path would shard by request across GPUs with no communication, so one "
              f"GPU's throughput is the per-GPU figure).", file=sys.stderr)
        sys.exit(2)

    import torch
    from top_selection_fm_amd import api
    from top_selection_fm_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    api.lib()
    if args.copy_calibration:
        copy_calibration(torch)
        return
    global CPU_BASELINES
    CPU_BASELINES = not args.no_cpu_baseline
    secondaries = {
        "mask": run_mask, "mask_shared_keys": lambda *a: run_mask(*a, shared=True),
        "mask_h128": lambda *a: run_mask(*a, heads=128),   # the retriever's head count
        "two_level": run_two_level, "prefill": run_prefill, "mode_a": run_mode_a,
        "encoder": run_encoder, "labels": run_labels}
    if args.only:
        if args.only not in secondaries:
            sys.exit(f"--only: one of {sorted(secondaries)}")
        print(json.dumps(secondaries[args.only](torch, api, W, args.steps, args.warmup)),
              flush=True)
        return

    log("headline: decode bf16 B=32 x 65536 ...")
    wl, h = run_decode(torch, api, W, args.steps, args.warmup)
    ms_step = h["graph_wall_s"] / args.steps * 1e3
    kern_ms = h["fused_b2b_ms"]
    digest = kernel_source_digest()
    achieved = h["alg_bytes"] / (kern_ms * 1e-3) / 1e9
    traffic = read_traffic("score_topk_decode_bf16_b32_s65536_counters.txt", digest)
    copy_gbs = stream_copy_gbs(torch)
    line = {
        "metric": "compressed-key entries scored+selected/sec (decode, bf16 keys)",
        "value": h["entries"] * args.steps / h["graph_wall_s"],
        "unit": "entries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_bf16_b32_s65536_top512", "requests": 32,
                   "entries_per_request": 65536, "page": 64, "heads": 64, "head_dim": 128,
                   "k": 512, "pool_replicas_rotated": 3,
                   "launch": "hip_graph, three steps (one per pool replica) a graph",
                   "call": "fm_index_topk (scoring and top-512 fused)"},
        "eager": {"ms_per_step": h["wall_s"] / args.steps * 1e3,
                  "value": h["entries"] * args.steps / h["wall_s"]},
        "graph_event_ms_per_step": h["graph_ms"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "fm_index_topk call: score_topk_bf16_kernel<4,16> (scoring + chunk "
                               "selection) then merge_chunks_kernel<1024,8> (row merge)",
                     "alg_bytes_per_launch": h["alg_bytes"], "avg_kernel_ms": kern_ms,
                     "timing": "events around back-to-back launches of the fused call",
                     "bracketed_ms": h["per"]["index_topk"],
                     "measured_copy_gbs": copy_gbs, "frac_of_measured_copy": achieved / copy_gbs},
        "two_call_path": h["two_call"],
        "kernels_ms": h["per"],
        "kernel_sources": digest,
    }
    if not args.headline_only:
        sec = []
        for name, fn in secondaries.items():
            log(f"secondary: {name} ...")
            try:
                sec.append(fn(torch, api, W, max(5, args.steps // 2), max(10, args.warmup)))
            except Exception as e:  # report and keep the headline
                sec.append(dict(workload=name, error=repr(e)))
            torch.cuda.empty_cache()
        line["secondary"] = sec
        # the MFMA-bound lines against the measured GEMM ceilings beside the published peaks
        ceil = vendor_gemm_tflops(torch)
        line["measured_mfma_ceilings"] = ceil
        f8, b16 = ceil.get("fp8_gemm_tflops"), ceil.get("bf16_gemm_tflops")
        for r in sec:
            wname = r.get("workload", "")
            if wname.startswith("prefill") and f8 and "mfma_tflops" in r:
                r["frac_of_vendor_fp8_gemm"] = r["mfma_tflops"] / f8
            if wname.endswith("shared_keys") and b16 and "mfma_tflops" in r:
                r["frac_of_vendor_bf16_gemm"] = r["mfma_tflops"] / b16
            if wname.startswith("query_encoder") and b16 and "t4096" in r:
                r["t4096"]["frac_of_vendor_bf16_gemm"] = r["t4096"]["mfma_tflops"] / b16
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(wl)
        line["cpu_baseline_single_thread_tiny"] = cpu_c1_single_thread(W)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
