"""Randomised parity sweep over small shapes (GPU).

Every entry point of the path on 64 seeded draws of batch size, heads, group size, block
size, ragged (and empty) request lengths, k, dtype and forcing flags, each held to the same
rules as the hand-picked cases in test_gpu_parity.py: metadata bit-exact, block and probe
scores within 1e-3 relative, selections equal up to near ties, attention (on the oracle's
selection, or on random selection rows) within the dtype's tolerance, and the fused calls'
selections (Quest and probe) bit-identical to the separate selection calls. The prefill importance has a sweep
of its own (24 draws of prompt lengths, padding, output stride, scale and dtype).
"""

import os

import numpy as np
import pytest
import torch

from tests.conftest import gpu_available
from tests.test_gpu_parity import (DEV, bits, check_attn, check_importance, check_scores, compare_probe,
                                   compare_quest, nbs_of, oracle_meta, random_selection, run_meta, run_select, say, tnp)
from top_kv_block_amd import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

# QS_SWEEP_DRAWS / QS_SWEEP_IMP_DRAWS widen the sweep for a longer run
N_DRAWS = int(os.environ.get("QS_SWEEP_DRAWS", "64"))


@pytest.fixture(scope="module")
def qs():
    from top_kv_block_amd import qsparse
    return qsparse


def draw(seed):
    """One random case: shapes, lengths, k, dtype and forcing from a seeded generator."""
    r = np.random.default_rng(7000 + seed)
    BS = int(r.choice([16, 32, 64, 128]))
    N = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 3, 4, 8]))
    B = int(r.integers(1, 5))
    max_nb = int(r.integers(1, 49))
    lens = []
    for _ in range(B):
        u = r.random()
        if u < 0.1:
            lens.append(0)                                   # empty request
        elif u < 0.2:
            lens.append(int(r.integers(1, BS + 1)))          # a single, maybe partial, block
        else:
            lens.append(int(r.integers(1, max_nb * BS + 1)))
    k = int(r.integers(1, 41))
    dtype = (torch.float32, torch.bfloat16, torch.float16)[int(r.integers(0, 3))]
    flags = int(r.integers(0, 4))
    tsmu = None
    if r.random() < 0.8:
        tsmu = [int(r.integers(-1, 2 * BS)) for _ in range(B)]
    n_probe = int(r.choice([1, 3, 8, 64]))
    return dict(B=B, H=N * G, N=N, BS=BS, lens=lens, k=k, dtype=dtype, flags=flags, tsmu=tsmu, n_probe=n_probe)


@pytest.mark.parametrize("seed", range(N_DRAWS))
def test_random_shapes_all_entry_points(qs, oracle, seed):
    c = draw(seed)
    B, H, N, BS, k, dtype, flags = c["B"], c["H"], c["N"], c["BS"], c["k"], c["dtype"], c["flags"]
    say(f"sweep seed={seed} B={B} H={H} N={N} BS={BS} lens={c['lens']} k={k} dtype={dtype} flags={flags} "
        f"tsmu={c['tsmu']} n_probe={c['n_probe']}")
    cover = None
    if c["tsmu"] is not None:
        cover = [max(0, L - max(t, 0)) for L, t in zip(c["lens"], c["tsmu"])]
    wl = W.random_case(100 + seed, B, H, N, BS, c["lens"], k=k, dtype=dtype, meta_cover=cover, tsmu=c["tsmu"],
                       flags=flags, with_importance=True)
    nbs = nbs_of(wl)

    # metadata (over the covered tokens), bit-exact, untouched rows keep the sentinel
    mx, mn = run_meta(qs, wl, sentinel=0.0)
    omx, omn = oracle_meta(oracle, wl, sentinel=0.0)
    assert np.array_equal(bits(tnp(mx)), bits(omx)) and np.array_equal(bits(tnp(mn)), bits(omn)), "metadata"

    # Quest selection
    sel, ns, sc = run_select(qs, wl, mx, mn)
    osel, ons, osc = oracle.block_select(wl.query, omx, omn, wl.meta_tables, wl.seq_lens, k, tsmu=wl.tsmu,
                                         flags=flags)
    mask = np.zeros_like(osc, dtype=bool)
    for b, nb in enumerate(nbs):
        mask[b, :, :nb] = ~np.isnan(osc[b, :, :nb])
    check_scores(tnp(sc), osc, mask)
    compare_quest(tnp(sel), tnp(ns), osel, ons, osc, nbs, k)

    # attention on the oracle's selection (one row per KV head)
    osel_t, ons_t = torch.from_numpy(osel), torch.from_numpy(ons)
    out = qs.qs_sparse_attn_decode(wl.query.to(DEV), wl.k_cache.to(DEV), wl.v_cache.to(DEV),
                                   wl.block_tables.to(DEV), wl.seq_lens.to(DEV), osel_t.to(DEV), ons_t.to(DEV))
    ref = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, osel, ons, N)
    args = (wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens)
    check_attn(out, ref, *args, osel, ons, N, "attention (Quest rows)")

    # attention on random per-query-head rows, with out-of-range entries
    rsel, rns = random_selection(seed, B, H, k, nbs)
    out = qs.qs_sparse_attn_decode(wl.query.to(DEV), wl.k_cache.to(DEV), wl.v_cache.to(DEV),
                                   wl.block_tables.to(DEV), wl.seq_lens.to(DEV), rsel.to(DEV), rns.to(DEV),
                                   sel_heads=H)
    ref = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, rsel, rns, H)
    check_attn(out, ref, *args, rsel, rns, H, "attention (random rows)")

    # fused selection + attention: the same selection as the selection call, bit for bit
    fsel = torch.full((B, N, k), -7, dtype=torch.int32, device=DEV)
    fns = torch.full((B, N), -7, dtype=torch.int32, device=DEV)
    ts = None if wl.tsmu is None else wl.tsmu.to(DEV)
    fout = qs.qs_select_attn_decode(wl.query.to(DEV), mx, mn, wl.meta_tables.to(DEV), wl.k_cache.to(DEV),
                                    wl.v_cache.to(DEV), wl.block_tables.to(DEV), wl.seq_lens.to(DEV), k,
                                    tokens_since_update=ts, flags=flags, selected=fsel, n_selected=fns)
    assert torch.equal(fsel, sel) and torch.equal(fns, ns), "fused selection differs from qs_block_select"
    gsel, gns = tnp(fsel), tnp(fns)
    ref = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, gsel, gns, N)
    check_attn(fout, ref, *args, gsel, gns, N, "fused attention")

    # probe selection (importance on, recency when the flags' low bit is set)
    pflags = W.RECENCY if flags & 1 else 0
    ps = torch.full((B, H, wl.mkbpr), float("inf"), device=DEV)
    psel, pns = qs.qs_probe_select(wl.query.to(DEV), wl.k_cache.to(DEV), wl.block_tables.to(DEV),
                                   wl.seq_lens.to(DEV), k, importance=wl.importance.to(DEV), n_probe=c["n_probe"],
                                   flags=pflags, probe_scores=ps)
    o = oracle.probe_select(wl.query, wl.k_cache, wl.block_tables, wl.seq_lens, k, N, importance=wl.importance,
                            n_probe=c["n_probe"], flags=pflags)
    pmask = np.zeros(o["probe"].shape, dtype=bool)
    for b, nb in enumerate(nbs):
        pmask[b, :, :nb] = True
    check_scores(tnp(ps), o["probe"], pmask)
    compare_probe(tnp(psel), tnp(pns), o, nbs, k)

    # fused probe selection + attention: the probe call's selection, bit for bit, and the
    # oracle's attention over it (one row per query head)
    fps = torch.full((B, H, k), -7, dtype=torch.int32, device=DEV)
    fpn = torch.full((B, H), -7, dtype=torch.int32, device=DEV)
    fo = qs.qs_probe_attn_decode(wl.query.to(DEV), wl.k_cache.to(DEV), wl.v_cache.to(DEV), wl.block_tables.to(DEV),
                                 wl.seq_lens.to(DEV), k, importance=wl.importance.to(DEV), n_probe=c["n_probe"],
                                 flags=pflags, selected=fps, n_selected=fpn)
    assert torch.equal(fps, psel) and torch.equal(fpn, pns), "fused probe selection differs from qs_probe_select"
    ref = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, tnp(psel),
                                    tnp(pns), H)
    check_attn(fo, ref, *args, tnp(psel), tnp(pns), H, "fused probe attention")

    # the same over an int8 copy of the cache (probes on the float K), for fp32 draws
    if dtype == torch.float32:
        k8, ks = W.quantize_rows_int8(wl.k_cache)
        v8, vs = W.quantize_rows_int8(wl.v_cache)
        fo8 = qs.qs_probe_attn_decode(wl.query.to(DEV), k8.to(DEV), v8.to(DEV), wl.block_tables.to(DEV),
                                      wl.seq_lens.to(DEV), k, importance=wl.importance.to(DEV), n_probe=c["n_probe"],
                                      flags=pflags, selected=fps, n_selected=fpn, k_scale=ks.to(DEV),
                                      v_scale=vs.to(DEV), probe_k=wl.k_cache.to(DEV))
        assert torch.equal(fps, psel) and torch.equal(fpn, pns), "int8 fused probe selection differs"
        ref = oracle.sparse_attn_decode(wl.query, k8, v8, wl.block_tables, wl.seq_lens, tnp(psel), tnp(pns), H,
                                        k_scale=ks, v_scale=vs)
        check_attn(fo8, ref, wl.query, k8, v8, wl.block_tables, wl.seq_lens, tnp(psel), tnp(pns), H,
                   "int8 fused probe attention", tol=2e-5)


IMP_DRAWS = int(os.environ.get("QS_SWEEP_IMP_DRAWS", "24"))


def draw_importance(seed):
    """One prefill-importance case: ragged (and empty) prompts of up to 1200 tokens, query
    rows padded past the longest prompt, an output stride shorter or longer than max_len,
    softmax scale default or drawn, dtype drawn; spans one to eight chunks of causal work."""
    r = np.random.default_rng(9000 + seed)
    BS = int(r.choice([16, 32, 64, 128]))
    N = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 3, 4]))
    B = int(r.integers(1, 4))
    lens = []
    for _ in range(B):
        u = r.random()
        lens.append(0 if u < 0.1 else int(r.integers(1, 65)) if u < 0.25 else int(r.integers(1, 1201)))
    top = max(max(lens), 1)
    max_len = top + int(r.choice([0, 0, int(r.integers(1, 200))]))
    stride = max(1, int(r.choice([max_len, max_len + int(r.integers(1, 100)), int(r.integers(1, max_len + 1))])))
    scale = 0.0 if r.random() < 0.5 else float(r.uniform(0.02, 0.3))
    dtype = (torch.float32, torch.bfloat16, torch.float16)[int(r.integers(0, 3))]
    return dict(B=B, H=N * G, N=N, BS=BS, lens=lens, max_len=max_len, stride=stride, scale=scale, dtype=dtype)


@pytest.mark.parametrize("seed", range(IMP_DRAWS))
def test_random_shapes_prefill_importance(qs, oracle, seed):
    c = draw_importance(seed)
    B, H, N, BS, lens, dtype = c["B"], c["H"], c["N"], c["BS"], c["lens"], c["dtype"]
    say(f"importance sweep seed={seed} B={B} H={H} N={N} BS={BS} lens={lens} max_len={c['max_len']} "
        f"stride={c['stride']} scale={c['scale']:.3f} dtype={dtype}")
    wl = W.random_case(200 + seed, B, H, N, BS, lens, k=1, dtype=dtype, with_v=False)
    q = W.prefill_queries(wl, 200 + seed, max_len=c["max_len"])
    imp, himp = qs.qs_prefill_importance(q.to(DEV), wl.k_cache.to(DEV), wl.block_tables.to(DEV), wl.seq_lens.to(DEV),
                                         softmax_scale=c["scale"], importance_stride=c["stride"], with_heads=True)
    torch.cuda.synchronize()
    oimp, ohimp = oracle.prefill_importance(q, wl.k_cache, wl.block_tables, wl.seq_lens, N, softmax_scale=c["scale"],
                                            stride=c["stride"])
    check_importance(tnp(imp), oimp, "importance")
    check_importance(tnp(himp), ohimp, "head importance")
    g = tnp(imp)
    for b, L in enumerate(lens):
        n = min(L, c["stride"])
        assert not g[b, n:].any(), "entries past the prompt must be zero"
        if L <= c["stride"] and L > 0:  # the whole prompt is in the output: each query row's weights sum to 1
            assert abs(g[b, :L].astype(np.float64).sum() - H * L) <= 1e-4 * H * L
