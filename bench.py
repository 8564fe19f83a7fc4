"""Decode-step benchmark of the sparse top-k KV-block attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload serving|long_context]

A step is one pass of the path over one batch: Quest block selection (grouped-query
scoring, top-k, sink/window forcing) followed by exact attention over the selected
blocks. The default workload is the large-batch serving decode: B=128, H=64, N=8, D=128,
BS=128, seq_len=32768, k=16, bf16 K/V (8 GiB each) in a shuffled paged pool; step s uses
query set s mod 4 and tokens_since_metadata_update = s mod 128. There the step is one
qs_select_attn_decode call (one kernel); the two-call path (qs_block_select, then
qs_sparse_attn_decode) is timed beside it. The full metadata rebuild and the refresh of
each request's newest block (the every-128-tokens update) are timed on their own, as is
the step rate with the caches flushed (1 GiB read) before each step.

Prints one JSON line: steps/s, ms/step, achieved algorithmic HBM GB/s of the step and of
its dominant kernel (HIP events around each launch on the launch stream), and the CPU
oracle's rate on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

PEAK_HBM_GBPS = 8000.0
METRIC = "sparse decode steps/s (select+attn) and achieved HBM GB/s vs MI355X peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cdiv(a, b):
    return -(-a // b)


def forced_count(L, BS, k, tsmu, flags):
    """Blocks the sink/window rule forces in (their metadata is not read)."""
    nb = cdiv(L, BS)
    if nb == 0 or tsmu < 0:
        return 0
    cnt, lo = 0, nb
    if flags & 2:
        n_meta = min(max((L - tsmu) // BS, 0), nb - 1)
        lo = max(n_meta, nb - k)
        cnt = nb - lo
    if (flags & 1) and cnt < k and lo > 0:
        cnt += 1
    return cnt


def step_bytes(wl, sel_h, ns_h, tsmu_h):
    """Algorithmic bytes of one step: what the method must read and write.

    select: max+min metadata rows of every non-forced candidate block (2*D*esize per
    (block, kv head)), the query, the indices written; attention: K and V rows of every
    valid token of every selected block for its kv head, the query, the output."""
    es = wl.k_cache.element_size()
    sl = wl.seq_lens.cpu().tolist()
    BS, N, D, H, B, k = wl.BS, wl.N, wl.D, wl.H, wl.B, wl.k
    sel_b = 0
    for b in range(B):
        nb = cdiv(sl[b], BS)
        cand = nb - forced_count(sl[b], BS, k, int(tsmu_h[b]), wl.flags)
        sel_b += cand * N * 2 * D * es
    sel_b += B * H * D * es + B * N * (k + 1) * 4
    att_b = 0
    for b in range(B):
        for n in range(N):
            for j in range(int(ns_h[b, n])):
                blk = int(sel_h[b, n, j])
                att_b += min(BS, sl[b] - blk * BS) * D * es * 2
    att_b += 2 * B * H * D * es + B * N * (k + 1) * 4
    return sel_b, att_b


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter summary,
    if it was taken on the current kernel sources (else None: the counters are stale)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    h = hashlib.sha256()
    for f in t["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return t["traffic_bytes"] if h.hexdigest() == t["source_sha256"] else None


def gather_requests(wl, reqs):
    """CPU copies of the sampled requests' blocks with remapped tables (marshalling)."""
    BS = wl.BS
    bt, mt = wl.block_tables.cpu(), wl.meta_tables.cpu()
    sl, msl = wl.seq_lens.cpu(), wl.meta_seq_lens.cpu()
    nbs = [cdiv(int(sl[b]), BS) for b in reqs]
    phys = torch.cat([bt[b, :nb].long() for b, nb in zip(reqs, nbs)]).to(wl.k_cache.device)
    kc, vc = wl.k_cache[phys].cpu(), wl.v_cache[phys].cpu()
    nt = torch.zeros((len(reqs), bt.shape[1]), dtype=torch.int32)
    nmt = torch.zeros((len(reqs), mt.shape[1]), dtype=torch.int32)
    off = moff = 0
    for j, nb in enumerate(nbs):
        nt[j, :nb] = torch.arange(off, off + nb, dtype=torch.int32)
        off += nb
        m = cdiv(nb, BS)
        nmt[j, :m] = torch.arange(moff, moff + m, dtype=torch.int32)
        moff += m
    return dict(kc=kc, vc=vc, bt=nt, mt=nmt, nmeta=max(1, moff), sl=sl[reqs].clone(), msl=msl[reqs].clone())


def run_cpu_baseline(wl, qsets, tsmu_tab, n_req, min_seconds):
    from oracle import oracle as O
    reqs = list(range(min(n_req, wl.B)))
    log(f"cpu baseline: gathering {len(reqs)} requests to the host")
    g = gather_requests(wl, reqs)
    mx, mn = O.build_metadata(g["kc"], g["bt"], g["msl"], g["mt"], g["nmeta"])   # untimed: not part of a step
    steps = 0
    t0 = time.perf_counter()
    while True:
        q = qsets[steps % qsets.shape[0]].cpu()[reqs]
        ts = tsmu_tab[steps % tsmu_tab.shape[0]].cpu()[reqs]
        sel, ns, _ = O.block_select(q, mx, mn, g["mt"], g["sl"], wl.k, tsmu=ts, flags=wl.flags)
        O.sparse_attn_decode(q, g["kc"], g["vc"], g["bt"], g["sl"], sel, ns, wl.N)
        steps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    per_sample_step = el / steps
    full_step = per_sample_step * wl.B / len(reqs)
    return {"value": 1.0 / full_step, "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(reqs)} of {wl.B} requests of the same workload, {steps} sample steps in {el:.1f} s, "
                      f"scaled by {wl.B}/{len(reqs)}; single-threaded C oracle (fp64)"}


def host_info():
    """The host the CPU baseline runs on: CPU model, logical CPUs, CPUs this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def _oracle_ms(fn, min_seconds):
    """Average ms of fn() over repeated calls totalling at least min_seconds (one warm call)."""
    fn()
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            return el * 1e3 / n


def cpu_baseline_rows(W, dev, min_seconds=0.5):
    """The oracle, single-threaded, on each of the other configurations (ms per step of the
    whole configuration; samples scaled as stated). Metadata the oracle's selection reads is
    built by the oracle beforehand and not counted, except where the build is the row."""
    from oracle import oracle as O
    rows = {}
    # the tiny fp32 workload, whole: Quest select + attention
    wl = W.tiny_needle()
    mx, mn = O.build_metadata(wl.k_cache, wl.block_tables, wl.seq_lens, wl.meta_tables, wl.num_meta_blocks)

    def tiny():
        sel, ns, _ = O.block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, wl.k)
        O.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, sel, ns, wl.N)
    rows[wl.name] = {"ms_per_step": round(_oracle_ms(tiny, min_seconds), 3), "sample": "whole workload"}

    # page-3-shaped select (bf16): 4 of its 20 requests (same shapes, drawn on the host), scaled by 5
    wl = W.page3_select(device="cpu", B=4)
    t_build = _oracle_ms(lambda: O.build_metadata(wl.k_cache, wl.block_tables, wl.seq_lens, wl.meta_tables,
                                                  wl.num_meta_blocks), min_seconds)
    mx, mn = O.build_metadata(wl.k_cache, wl.block_tables, wl.seq_lens, wl.meta_tables, wl.num_meta_blocks)
    t_sel = _oracle_ms(lambda: O.block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, wl.k), min_seconds)
    rows["page3_select_b20_l16384_bf16"] = {"select_ms": round(t_sel * 5, 3), "metadata_build_ms": round(t_build * 5, 3),
                                            "sample": "4 of 20 requests, scaled by 5"}

    # page-1 probe selection + fp32 / int8 attention, k = 1 .. 32, whole workload
    wl = W.page1_probe()
    sweep = {}
    for kk in (1, 2, 4, 8, 16, 32):
        o = O.probe_select(wl.query, wl.k_cache, wl.block_tables, wl.seq_lens, kk, wl.N, importance=wl.importance,
                           n_probe=8, flags=O.RECENCY)

        def step(int8, kk=kk):
            r = O.probe_select(wl.query, wl.k_cache, wl.block_tables, wl.seq_lens, kk, wl.N,
                               importance=wl.importance, n_probe=8, flags=O.RECENCY)
            if int8:
                O.sparse_attn_decode(wl.query, wl.k_i8, wl.v_i8, wl.block_tables, wl.seq_lens, r["selected"],
                                     r["n_selected"], wl.H, k_scale=wl.k_scale, v_scale=wl.v_scale)
            else:
                O.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, r["selected"],
                                     r["n_selected"], wl.H)
        sweep[f"k{kk}"] = {"step_fp32_ms": round(_oracle_ms(lambda: step(False), min_seconds / 2), 3),
                           "step_int8_ms": round(_oracle_ms(lambda: step(True), min_seconds / 2), 3),
                           "selected_per_head": int(o["n_selected"][0, 0])}
    rows["page1_probe_b1_h16_l4096_k_sweep"] = {"by_k": sweep, "sample": "whole workload"}

    # long-context decode: 2 of its 8 requests (gathered from the GPU-drawn pools), scaled by 4
    wl = W.long_context(device=dev)
    g = gather_requests(wl, [0, 1])
    q = wl.query.cpu()[[0, 1]]
    ts = wl.tsmu.cpu()[[0, 1]]
    del wl
    torch.cuda.empty_cache()
    mx, mn = O.build_metadata(g["kc"], g["bt"], g["msl"], g["mt"], g["nmeta"])

    def lc():
        sel, ns, _ = O.block_select(q, mx, mn, g["mt"], g["sl"], 64, tsmu=ts, flags=3)
        O.sparse_attn_decode(q, g["kc"], g["vc"], g["bt"], g["sl"], sel, ns, 8)
    rows["long_context_b8_l8k_128k_bf16"] = {"ms_per_step": round(_oracle_ms(lc, min_seconds) * 4, 3),
                                             "sample": f"requests 0 and 1 (lengths {g['sl'].tolist()}), scaled by 4"}
    return rows


def _timed(fn, reps, stream, rounds=3):
    """Average ms of fn() over reps back-to-back calls on the stream (after one warm call);
    the median of `rounds` such rounds."""
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / reps)
    return sorted(ts)[len(ts) // 2]


def _graph_us(fn, reps, stream):
    """Average us of fn() replayed from one captured HIP graph of ``reps`` calls (the GPU
    time of the call without the host's launch and marshalling cost)."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for _ in range(reps):
                fn()
    stream.wait_stream(cs)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (3 * reps)


def other_workloads(qs, W, dev, stream, reps=50):
    """The other configurations of the path, each timed on its own (ms per call and
    algorithmic GB/s); they are parity-test cases too, these are measurements only."""
    res = {}

    def gbps(nbytes, ms):
        return round(nbytes / (ms * 1e-3) / 1e9, 1)

    def meta_buf(wl):
        return qs.alloc_metadata_pools(wl.num_meta_blocks, wl.BS, wl.N, wl.D, dtype=wl.k_cache.dtype, device=dev)

    # the tiny fp32 workload: Quest select + attention
    wl = W.tiny_needle().to(dev)
    mx, mn = meta_buf(wl)
    qs.qs_build_metadata(wl.k_cache, wl.block_tables, wl.seq_lens, wl.meta_tables, mx, mn)
    sel, ns = qs.qs_block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, wl.k)
    t_sel = _timed(lambda: qs.qs_block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, wl.k, selected=sel,
                                              n_selected=ns), reps, stream)
    t_att = _timed(lambda: qs.qs_sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens,
                                                    sel, ns), reps, stream)
    out1 = torch.empty_like(wl.query)
    t_fused = _timed(lambda: qs.qs_select_attn_decode(wl.query, mx, mn, wl.meta_tables, wl.k_cache, wl.v_cache,
                                                      wl.block_tables, wl.seq_lens, wl.k, out=out1), reps, stream)
    g_fused = _graph_us(lambda: qs.qs_select_attn_decode(wl.query, mx, mn, wl.meta_tables, wl.k_cache, wl.v_cache,
                                                         wl.block_tables, wl.seq_lens, wl.k, out=out1), reps, stream)
    res[wl.name] = {"select_us": round(t_sel * 1e3, 2), "attention_us": round(t_att * 1e3, 2),
                    "step_us": round((t_sel + t_att) * 1e3, 2),
                    "fused_step_us": round(t_fused * 1e3, 2), "fused_step_graph_us": round(g_fused, 2),
                    "note": "latency-bound (0.33 MB a step); *_graph_us: the call replayed from a HIP graph "
                            "(GPU time without host launch cost)"}
    del wl, mx, mn

    # page-3-shaped Quest select, bf16 and fp16 (the page's metadata example is
    # fp16); metadata build timed too
    for dt in (torch.bfloat16, torch.float16):
        wl = W.page3_select(device=dev, dtype=dt)
        mx, mn = meta_buf(wl)
        t_build = _timed(lambda: qs.qs_build_metadata(wl.k_cache, wl.block_tables, wl.seq_lens, wl.meta_tables, mx,
                                                      mn), 10, stream)
        tz = torch.zeros(wl.B, dtype=torch.int32, device=dev)
        sel = torch.empty((wl.B, wl.N, wl.k), dtype=torch.int32, device=dev)
        ns = torch.empty((wl.B, wl.N), dtype=torch.int32, device=dev)
        t0 = _timed(lambda: qs.qs_block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, wl.k, selected=sel,
                                               n_selected=ns), reps, stream)
        t1 = _timed(lambda: qs.qs_block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, wl.k,
                                               tokens_since_update=tz, flags=3, selected=sel, n_selected=ns),
                    reps, stream)
        g0 = _graph_us(lambda: qs.qs_block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, wl.k, selected=sel,
                                                  n_selected=ns), reps, stream)
        es = 2
        sel_bytes = wl.B * wl.N * 128 * 2 * wl.D * es + wl.B * wl.H * wl.D * es
        build_bytes = wl.k_cache.numel() * es + wl.num_meta_blocks * wl.BS * wl.N * wl.D * es * 2
        res[wl.name] = {"select_us": round(t0 * 1e3, 2), "select_gbps": gbps(sel_bytes, t0),
                        "select_graph_us": round(g0, 2), "select_window_us": round(t1 * 1e3, 2),
                        "metadata_build_us": round(t_build * 1e3, 2),
                        "metadata_build_gbps": gbps(build_bytes, t_build),
                        "note": "select_graph_us: the select replayed from a HIP graph (GPU time without host "
                                "launch cost)"}
        del wl, mx, mn

    # page-1 probe selection + fp32 / int8 attention, k = 1 .. 32
    wl = W.page1_probe().to(dev)
    sweep = {}
    for kk in (1, 2, 4, 8, 16, 32):
        psel, pns = qs.qs_probe_select(wl.query, wl.k_cache, wl.block_tables, wl.seq_lens, kk,
                                       importance=wl.importance, n_probe=8, flags=qs.QS_RECENCY)
        pout = torch.empty_like(wl.query)

        def probe():
            qs.qs_probe_select(wl.query, wl.k_cache, wl.block_tables, wl.seq_lens, kk, importance=wl.importance,
                               n_probe=8, flags=qs.QS_RECENCY, selected=psel, n_selected=pns)

        def att(int8):
            if int8:
                qs.qs_sparse_attn_decode(wl.query, wl.k_i8, wl.v_i8, wl.block_tables, wl.seq_lens, psel, pns,
                                         sel_heads=wl.H, k_scale=wl.k_scale, v_scale=wl.v_scale, out=pout)
            else:
                qs.qs_sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, psel, pns,
                                         sel_heads=wl.H, out=pout)

        def fused(int8):
            if int8:
                qs.qs_probe_attn_decode(wl.query, wl.k_i8, wl.v_i8, wl.block_tables, wl.seq_lens, kk,
                                        importance=wl.importance, n_probe=8, flags=qs.QS_RECENCY, out=pout,
                                        probe_k=wl.k_cache, k_scale=wl.k_scale, v_scale=wl.v_scale)
            else:
                qs.qs_probe_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, kk,
                                        importance=wl.importance, n_probe=8, flags=qs.QS_RECENCY, out=pout)

        row = {"probe_select_us": round(_timed(probe, reps, stream) * 1e3, 2)}
        for int8, tag in ((False, "fp32"), (True, "int8")):
            row[f"attention_{tag}_us"] = round(_timed(lambda: att(int8), reps, stream) * 1e3, 2)
            row[f"step_{tag}_us"] = round(_timed(lambda: (probe(), att(int8)), reps, stream) * 1e3, 2)
            row[f"fused_step_{tag}_us"] = round(_timed(lambda: fused(int8), reps, stream) * 1e3, 2)
            row[f"fused_step_{tag}_graph_us"] = round(_graph_us(lambda: fused(int8), reps, stream), 2)
        sweep[f"k{kk}"] = row
    probe_bytes = wl.N * 128 * 8 * wl.D * 4 + 4096 * 4 + wl.H * wl.D * 4
    k32 = sweep["k32"]
    res["page1_probe_b1_h16_l4096_k_sweep"] = {
        "by_k": sweep, "probe_select_gbps_k32": gbps(probe_bytes, k32["probe_select_us"] * 1e-3),
        "note": "latency-bound (a few MB a step); step_*_us: qs_probe_select + qs_sparse_attn_decode back to back; "
                "fused_step_*_us: one qs_probe_attn_decode call (int8: probe on the float K, attention on the "
                "int8 copy); *_graph_us: replayed from a HIP graph (GPU time without host launch cost)"}
    del wl

    # the prefill that produces the probe workload's importance (fp32 inputs): one causal QK^T pass
    # on the matrix cores that also stores the scores' causal 16x16 tiles, then a pass that streams
    # them back for the column sums; algorithmic flops: H heads x L(L+1)/2 causal dots x 2D
    wl, pq = W.page1_probe_prefill()
    wl, pq = wl.to(dev), pq.to(dev)
    imp = torch.empty((wl.B, int(wl.seq_lens.max())), dtype=torch.float32, device=dev)
    t_imp = _timed(lambda: qs.qs_prefill_importance(pq, wl.k_cache, wl.block_tables, wl.seq_lens, importance=imp),
                   10, stream)
    L = int(wl.seq_lens.max())
    method_flops = wl.H * L * (L + 1) * wl.D          # one causal Q K^T: H * L(L+1)/2 dots of 2D flops
    t16 = (L + 15) // 16
    score_bytes = wl.B * wl.H * t16 * (t16 + 1) // 2 * 1024   # stored causal 16x16 fp32 tiles
    res["page1_prefill_importance_b1_h16_l4096_fp32"] = {
        "us": round(t_imp * 1e3, 2), "method_gflop": round(method_flops / 1e9, 2),
        "tflops": round(method_flops / (t_imp * 1e-3) / 1e12, 2),
        "mfma_fp32_peak_tflops": 157.3, "frac": round(method_flops / (t_imp * 1e-3) / 1e12 / 157.3, 4),
        "stored_score_mb": round(score_bytes / 1e6, 1),
        "note": "B=1, L=4096, H=16, N=8; frac counts the method's own work (one causal QK^T); the call also "
                "writes the scores' causal tiles once and reads them back once (stored_score_mb each way)"}
    del wl, pq, imp

    # long-context paged decode, bf16 (rows split over workgroups + combine)
    wl = W.long_context(device=dev)
    mx, mn = meta_buf(wl)
    qs.qs_build_metadata(wl.k_cache, wl.block_tables, wl.meta_seq_lens, wl.meta_tables, mx, mn)
    sel = torch.empty((wl.B, wl.N, wl.k), dtype=torch.int32, device=dev)
    ns = torch.empty((wl.B, wl.N), dtype=torch.int32, device=dev)
    out = torch.empty((wl.B, wl.H, wl.D), dtype=torch.bfloat16, device=dev)

    def c4_select():
        qs.qs_block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, wl.k, tokens_since_update=wl.tsmu,
                           flags=wl.flags, selected=sel, n_selected=ns)

    def c4_attend():
        qs.qs_sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, sel, ns, out=out)

    t_s = _timed(c4_select, reps, stream)
    t_a = _timed(c4_attend, reps, stream)
    t_step = _timed(lambda: (c4_select(), c4_attend()), reps, stream)
    t_fused = _timed(lambda: qs.qs_select_attn_decode(wl.query, mx, mn, wl.meta_tables, wl.k_cache, wl.v_cache,
                                                      wl.block_tables, wl.seq_lens, wl.k,
                                                      tokens_since_update=wl.tsmu, flags=wl.flags, out=out,
                                                      selected=sel, n_selected=ns), reps, stream)
    sb, ab = step_bytes(wl, sel.cpu(), ns.cpu(), wl.tsmu.cpu())
    res[wl.name] = {
        "step_us": round(t_step * 1e3, 2), "steps_per_s": round(1000.0 / t_step, 1),
        "fused_step_us": round(t_fused * 1e3, 2), "fused_steps_per_s": round(1000.0 / t_fused, 1),
        "step_bytes": int(sb + ab), "step_gbps": gbps(sb + ab, t_step),
        "select_us": round(t_s * 1e3, 2), "select_gbps": gbps(sb, t_s),
        "attention_us": round(t_a * 1e3, 2), "attention_gbps": gbps(ab, t_a),
        "needle_recall": sum(int((t // wl.BS) in set(sel[b, n, :ns[b, n]].cpu().tolist()))
                             for b, t in wl.needles for n in range(wl.N)) / (wl.B * wl.N)}
    del wl, mx, mn
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="serving", choices=["serving", "long_context"])
    ap.add_argument("--cpu-sample", type=int, default=4, help="requests in the CPU-baseline sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--path", choices=["fused", "separate"], default=None,
                    help="step as one qs_select_attn_decode call (default for the serving workload) or as "
                         "qs_block_select + qs_sparse_attn_decode (default for the long-context workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flushed-steps", type=int, default=32,
                    help="steps timed one by one after a 1 GiB cache flush each (0: skip)")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip timing the other configurations (tiny, page-3 select, probe, long context)")
    ap.add_argument("--graph-steps", type=int, default=128,
                    help="steps captured in one HIP graph for the replay figure (0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=1024,
                    help="size of the plain device copy timed beside the step (0 = skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path has no cross-GPU step (each GPU runs these kernels "
              "on its own share of the requests); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    from top_kv_block_amd import qsparse as qs
    from top_kv_block_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"generating {args.workload} on the GPU")
    wl = W.serving(device=dev) if args.workload == "serving" else W.long_context(device=dev)
    qsets = wl.extra.get("query_sets", wl.query[None])
    B, H, N, D, BS, k = wl.B, wl.H, wl.N, wl.D, wl.BS, wl.k
    if args.workload == "serving":
        tsmu_tab = (torch.arange(128, dtype=torch.int32, device=dev)[:, None] % 128).repeat(1, B).contiguous()
    else:
        tsmu_tab = wl.tsmu[None].contiguous()
    # metadata pools placed as the library recommends (min 256 B past a 1 KiB multiple from
    # max); the workload's K and V pools are placed the same way (workloads.paired_pools)
    mx, mn = qs.alloc_metadata_pools(wl.num_meta_blocks, BS, N, D, dtype=wl.k_cache.dtype, device=dev)
    sel = torch.empty((B, N, k), dtype=torch.int32, device=dev)
    ns = torch.empty((B, N), dtype=torch.int32, device=dev)
    out = torch.empty((B, H, D), dtype=wl.query.dtype, device=dev)
    ws_sel = torch.zeros(qs.block_select_workspace_bytes(B, N, BS, wl.mmbpr), dtype=torch.uint8, device=dev)
    ws_att = torch.zeros(qs.sparse_attn_workspace_bytes(B, H, N, D, N, k), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def rebuild():
        qs.qs_build_metadata(wl.k_cache, wl.block_tables, wl.meta_seq_lens, wl.meta_tables, mx, mn)

    def select_on(m):
        def select(s):
            qs.qs_block_select(qsets[s % qsets.shape[0]], mx, m, wl.meta_tables, wl.seq_lens, k,
                               tokens_since_update=tsmu_tab[s % tsmu_tab.shape[0]], flags=wl.flags, selected=sel,
                               n_selected=ns, workspace_buf=ws_sel)
        return select

    def attend_on(v):
        def attend(s):
            qs.qs_sparse_attn_decode(qsets[s % qsets.shape[0]], wl.k_cache, v, wl.block_tables, wl.seq_lens,
                                     sel, ns, sel_heads=N, out=out, workspace_buf=ws_att)
        return attend

    select, attend = select_on(mn), attend_on(wl.v_cache)

    log("metadata build")
    rebuild()
    torch.cuda.synchronize()
    # metadata rebuild, timed on its own
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        rebuild()
    e1.record(stream)
    torch.cuda.synchronize()
    rebuild_ms = e0.elapsed_time(e1) / 3
    es = wl.k_cache.element_size()
    mlens = [max(int(L), 0) for L in wl.meta_seq_lens.cpu().tolist()]
    meta_bytes = sum(L * N * D * es for L in mlens) + \
        sum(cdiv(cdiv(L, BS), BS) * BS * N * D * es * 2 for L in mlens)   # K read + max/min rows written

    # refresh of the newest block of every request (the every-128-tokens metadata update)
    first_blk = torch.tensor([max(cdiv(L, BS) - 1, 0) for L in mlens], dtype=torch.int32, device=dev)

    def refresh():
        qs.qs_update_metadata(wl.k_cache, wl.block_tables, wl.meta_seq_lens, first_blk, 1, wl.meta_tables, mx, mn)

    refresh()
    e0.record(stream)
    for _ in range(20):
        refresh()
    e1.record(stream)
    torch.cuda.synchronize()
    refresh_us = e0.elapsed_time(e1) / 20 * 1e3
    refresh_bytes = sum((L - (cdiv(L, BS) - 1) * BS) * N * D * es + N * D * es * 2 for L in mlens if L > 0)

    copy_gbps = None
    if args.copy_calibration_mib > 0:
        # a plain device-to-device copy of known size: the bandwidth a simple streaming
        # kernel reaches on this machine, and the reference the HBM byte counters are scaled by
        nbytes = args.copy_calibration_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(5):
            dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_gbps = 2 * nbytes * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
        del src, dst

    ws_fused = torch.zeros(qs.select_attn_workspace_bytes(B, H, N, BS, wl.mmbpr, k, qs.QS_BF16), dtype=torch.uint8,
                           device=dev)

    def fused_on(v, m):
        def fused(s):
            # the fused entry point: selection kept on chip and attention in one launch when
            # the rows allow it (the serving shape does); the selection is still written out
            qs.qs_select_attn_decode(qsets[s % qsets.shape[0]], mx, m, wl.meta_tables, wl.k_cache, v,
                                     wl.block_tables, wl.seq_lens, k,
                                     tokens_since_update=tsmu_tab[s % tsmu_tab.shape[0]], flags=wl.flags, out=out,
                                     selected=sel, n_selected=ns, workspace_buf=ws_fused)
        return fused

    def separate_on(v, m):
        sel_f, att_f = select_on(m), attend_on(v)

        def separate(s):
            sel_f(s)
            att_f(s)
        return separate

    fused, separate = fused_on(wl.v_cache, mn), separate_on(wl.v_cache, mn)

    path = args.path or ("fused" if args.workload == "serving" else "separate")
    step = fused if path == "fused" else separate
    other = separate if path == "fused" else fused

    log(f"warmup {args.warmup} steps of each path")
    for s in range(args.warmup):
        fused(s)
        separate(s)
    torch.cuda.synchronize()

    K = args.steps

    def time_steps(fn):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for s in range(K):
            fn(s)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    # (1) the step rate: K steps back to back, events only around the whole region
    log(f"timing {K} steps ({path} path)")
    total_ms = time_steps(step)
    log(f"timing {K} steps (the other path)")
    other_ms = time_steps(other) / K

    # (1b) the same steps with the caches flushed before each one: reading a 1 GiB buffer
    # evicts L2 and the 256 MB last-level cache, so nothing of the step's inputs is cache
    # resident (a read, not a fill, so no dirty lines are left to be written back during
    # the step); events around each step
    flushed = None
    if args.flushed_steps > 0:
        log(f"timing {args.flushed_steps} steps after a cache flush each")
        junk = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        acc = torch.zeros((), dtype=torch.float32, device=dev)
        fe = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.flushed_steps)]
        for s in range(args.flushed_steps):
            acc += junk.sum()
            fe[s][0].record(stream)
            step(s)
            fe[s][1].record(stream)
        torch.cuda.synchronize()
        f_ms = float(np.mean([a.elapsed_time(b) for a, b in fe]))
        flushed = {"steps_per_s": round(1000.0 / f_ms, 3), "step_us": round(f_ms * 1e3, 2),
                   "steps": args.flushed_steps, "flush": "1 GiB read before each step; events around each step"}
        del junk

    # (2) per-launch durations: the same K steps with HIP events around every launch, on
    # the stream the kernels run on (the events themselves add a little time between
    # launches, so the step rate above is taken without them)
    log(f"timing {K} steps with per-launch events")

    def per_launch(fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        torch.cuda.synchronize()
        for s in range(K):
            ev[s][0].record(stream)
            fn(s)
            ev[s][1].record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev])

    fused_ms = per_launch(fused)
    select_ms = per_launch(select)
    attn_ms = per_launch(attend)

    # (3) the same steps replayed from one captured HIP graph (no host launch overhead)
    graph_ms = None
    if args.graph_steps > 0:
        log(f"capturing {args.graph_steps} steps in a HIP graph")
        gs = args.graph_steps
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(stream)
        with torch.cuda.stream(cs):
            with torch.cuda.graph(g, stream=cs):
                for s in range(gs):
                    step(s)
        stream.wait_stream(cs)
        g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(1, K // gs)
        g0.record(stream)
        for _ in range(reps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / (reps * gs)

    # (4) pool placement: the same steps with the V and min pools copied to addresses that
    # agree with K's and max's modulo 1 KiB, as separately allocated pools (or the two halves
    # of one [2, ...] pool) usually do; the step above uses the placement the library
    # recommends (qs.alloc_kv_pools, qs.alloc_metadata_pools)
    def same_phase_copy(t, ref):
        nbytes = t.numel() * t.element_size()
        buf = torch.empty(nbytes + 1024, dtype=torch.uint8, device=dev)
        o = (ref.data_ptr() - buf.data_ptr()) % 1024
        c = buf[o:o + nbytes].view(t.dtype).view(t.shape)
        c.copy_(t)
        return c

    log("timing the step with the V and min pools at K's and max's address phase")
    v_al, mn_al = same_phase_copy(wl.v_cache, wl.k_cache), same_phase_copy(mn, mx)
    step_al = fused_on(v_al, mn_al) if path == "fused" else separate_on(v_al, mn_al)
    for s in range(args.warmup):
        step_al(s)
    aligned_ms = time_steps(step_al) / K
    placement = {
        "used": "V pool 256 B past a 1 KiB multiple from the K pool, min pool likewise from max "
                "(the layout of qs.alloc_kv_pools / qs.alloc_metadata_pools); value is measured on it",
        "v_minus_k_mod_1KiB": (wl.v_cache.data_ptr() - wl.k_cache.data_ptr()) % 1024,
        "min_minus_max_mod_1KiB": (mn.data_ptr() - mx.data_ptr()) % 1024,
        "same_phase_pools": {"steps_per_s": round(1000.0 / aligned_ms, 3), "ms_per_step": round(aligned_ms, 5),
                             "v_minus_k_mod_1KiB": (v_al.data_ptr() - wl.k_cache.data_ptr()) % 1024,
                             "min_minus_max_mod_1KiB": (mn_al.data_ptr() - mx.data_ptr()) % 1024},
    }
    del v_al, mn_al, step_al
    torch.cuda.empty_cache()

    # replay the selections of the timed steps to count their algorithmic bytes
    log("counting algorithmic bytes of the timed steps")
    sel_bytes = att_bytes = 0
    sample_steps = sorted(set([0, 1, 2, 3] + list(range(0, K, max(1, K // 16)))))
    for s in sample_steps:
        select(s)
        torch.cuda.synchronize()
        sb, ab = step_bytes(wl, sel.cpu(), ns.cpu(), tsmu_tab[s % tsmu_tab.shape[0]].cpu())
        sel_bytes += sb
        att_bytes += ab
    sel_bytes /= len(sample_steps)
    att_bytes /= len(sample_steps)
    ms_per_step = total_ms / K
    step_gbps = (sel_bytes + att_bytes) / (ms_per_step * 1e-3) / 1e9
    if path == "fused":
        # one kernel per step in the serving shape: select_attn_mfma_kernel moves the whole step
        dom_kernel, dom_ms, dom_bytes = "select_attn_mfma_kernel (qs_select_attn_decode)", fused_ms, sel_bytes + att_bytes
    else:
        # the events bracket the whole qs_sparse_attn_decode call: with split rows (the
        # long-context shape) that is attn_mfma_kernel plus attn_combine_kernel
        dom_kernel, dom_ms, dom_bytes = ("attn_mfma_kernel + attn_combine_kernel (qs_sparse_attn_decode)", attn_ms,
                                         att_bytes)
    dom_avg_ms = float(dom_ms.mean())
    dom_gbps = dom_bytes / (dom_avg_ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(1000.0 / ms_per_step, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "H": H, "N": N, "D": D, "block_size": BS,
                   "seq_len": int(wl.seq_lens.max()), "k": k, "flags": "sink+window",
                   "query_sets": int(qsets.shape[0]),
                   "path": "qs_select_attn_decode" if path == "fused" else "qs_block_select + qs_sparse_attn_decode"},
        "step_bytes": int(sel_bytes + att_bytes),
        "step_gbps": round(step_gbps, 1),
        "step_hbm_frac": round(step_gbps / PEAK_HBM_GBPS, 4),
        "select_bytes": int(sel_bytes),
        "attention_bytes": int(att_bytes),
        "other_path": {"path": "qs_block_select + qs_sparse_attn_decode" if path == "fused" else "qs_select_attn_decode",
                       "steps_per_s": round(1000.0 / other_ms, 3), "ms_per_step": round(other_ms, 5)},
        "graph_replay_steps_per_s": None if graph_ms is None else round(1000.0 / graph_ms, 3),
        "fused_call_avg_us": round(float(fused_ms.mean()) * 1000, 3),
        "select_avg_us": round(float(select_ms.mean()) * 1000, 3),
        "select_gbps": round(sel_bytes / (float(select_ms.mean()) * 1e-3) / 1e9, 1),
        "attention_avg_us": round(float(attn_ms.mean()) * 1000, 3),
        "attention_gbps": round(att_bytes / (float(attn_ms.mean()) * 1e-3) / 1e9, 1),
        "device_copy_gbps": None if copy_gbps is None else round(copy_gbps, 1),
        "metadata_rebuild_ms": round(rebuild_ms, 4),
        "metadata_rebuild_gbps": round(meta_bytes / (rebuild_ms * 1e-3) / 1e9, 1),
        "steps_per_s_with_rebuild_every_128": round(128.0 / (128 * ms_per_step + rebuild_ms) * 1000.0, 3),
        "metadata_refresh_us": round(refresh_us, 2),
        "metadata_refresh_gbps": round(refresh_bytes / (refresh_us * 1e-6) / 1e9, 1),
        "steps_per_s_with_refresh_every_128": round(128.0 / (128 * ms_per_step + refresh_us * 1e-3) * 1000.0, 3),
        "flushed": flushed,
        "pool_placement": placement,
        "roofline": {"kernel": dom_kernel, "bound": "hbm",
                     "achieved": round(dom_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(dom_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic(dom_kernel.split()[0], wl.name),
                     "avg_launch_us": round(dom_avg_ms * 1000, 3), "bytes_per_launch": int(dom_bytes)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = run_cpu_baseline(wl, qsets, tsmu_tab, args.cpu_sample, args.cpu_seconds)
        result["host"] = host_info()
    if not args.no_other_workloads:
        del wl, qsets, mx, mn
        torch.cuda.empty_cache()
        log("timing the other workloads")
        result["other_workloads"] = other_workloads(qs, W, dev, stream)
        if not args.no_cpu_baseline:
            log("cpu baseline of the other workloads")
            result["cpu_baseline_workloads"] = cpu_baseline_rows(W, dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
