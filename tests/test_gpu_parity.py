"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same
seeded inputs.

Bars (the tolerance contract of the path):
  * metadata max/min: bit-exact, including the +0.0 tail rows and untouched rows;
  * block / probe scores: |gpu - oracle| <= 1e-3 * max(|oracle|, 1e-3 * max_row |oracle|);
  * selections: forced and importance picks exact; the rest equal wherever the oracle's
    k-th and (k+1)-th fill scores differ by more than 1e-3 relative, otherwise differing
    only in blocks whose oracle score is within 1e-3 relative of the k-th;
  * attention (on the oracle's selection): max abs error <= 1e-4 (fp32 out), <= 2e-2
    (bf16 out); the int8 path (exact int32 dots) also within 2e-5 for fp32 queries. A
    16-bit query over a KV cache of the same type is also held, element by element, to the
    rounding bound of tests/bounds.py (the operand-format rounding of the weights and of
    the output), which rejects a dropped block or 32-token chunk that 2e-2 alone accepts.
"""

import math
import os
import sys

import numpy as np
import pytest
import torch

from tests.bounds import attn16_bound, check_attn16
from tests.conftest import gpu_available
from tests.helpers import as_sets, cdiv, check_selection_rows, near_tie_equal
from top_kv_block_amd import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

DEV = "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def qs():
    from top_kv_block_amd import qsparse
    return qsparse


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint8)


def tnp(t):
    """numpy copy of a device tensor; bf16 as uint16 bits."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# ------------------------------------------------------------------------------------------
# comparison helpers
# ------------------------------------------------------------------------------------------

def check_scores(gpu, ref, valid_mask, rel=1e-3):
    g = gpu[valid_mask].astype(np.float64)
    o = ref[valid_mask]
    if o.size == 0:
        return
    floor = 1e-3 * np.max(np.abs(o))
    if floor == 0.0:  # every reference score is zero (e.g. metadata over no token): exact
        assert np.all(g == o), f"scores should all be zero: {g[g != o][:4]}"
        return
    err = np.abs(g - o) / np.maximum(np.abs(o), floor)
    assert np.all(err <= rel), f"score rel err {err.max():.3e}"


def compare_quest(gsel, gns, osel, ons, osc, nbs, k):
    check_selection_rows(gsel, gns, k)
    B, N = gns.shape
    np.testing.assert_array_equal(gns, ons)
    near = 0
    for b in range(B):
        nb = nbs[b]
        for n in range(N):
            got = set(gsel[b, n, :gns[b, n]].tolist())
            want = set(osel[b, n, :ons[b, n]].tolist())
            sc = osc[b, n, :nb]
            fixed = {i for i in range(nb) if np.isnan(sc[i])}
            fill = {i: sc[i] for i in range(nb) if not np.isnan(sc[i])}
            ok, why = near_tie_equal(got, want, fill, fixed)
            assert ok, f"(b={b}, n={n}) {why}: gpu={sorted(got)} oracle={sorted(want)}"
            near += why == "near tie"
    return near


def compare_probe(gsel, gns, o, nbs, k):
    check_selection_rows(gsel, gns, k)
    np.testing.assert_array_equal(gns, o["n_selected"])
    B, H = gns.shape
    for b in range(B):
        nb = nbs[b]
        for h in range(H):
            got = set(gsel[b, h, :gns[b, h]].tolist())
            want = set(o["selected"][b, h, :o["n_selected"][b, h]].tolist())
            kind = o["kind"][b, h]
            imp = {i for i in range(nb) if kind[i] == 1}
            pr = o["probe"][b, h]
            fill = {i: pr[i] for i in range(nb) if i not in imp}
            pre = [i for i in range(nb) if kind[i] in (2, 4)]
            if got != want:
                assert imp <= got, f"(b={b}, h={h}) importance picks differ"
                s_k = min(pr[i] for i in pre)
                tol = 1e-3 * max(abs(s_k), 1e-30)
                for i in got ^ want:
                    assert i in fill and abs(fill[i] - s_k) <= tol, \
                        f"(b={b}, h={h}) block {i}: gpu={sorted(got)} oracle={sorted(want)}"


def attn_tol(q_dtype):
    return {torch.bfloat16: 2e-2, torch.float16: 5e-3}.get(q_dtype, 1e-4)


def check_attn(out, ref, q, kc, vc, bt, sl, sel, ns, sel_heads, what, tol=None):
    """Attention output against the oracle's over the same selection: the contract's
    absolute tolerance for the output dtype (or ``tol``) and, for a 16-bit query over a KV
    cache of the same type, the per-element rounding bound too. Logs the observed error."""
    got = out.float().cpu().numpy().astype(np.float64) if isinstance(out, torch.Tensor) else out
    if q.dtype in (torch.bfloat16, torch.float16) and kc.dtype == q.dtype:
        bound = attn16_bound(q, kc, vc, bt, sl, sel, ns, sel_heads, ref, q.dtype)
        return check_attn16(got, ref, bound, what, contract=attn_tol(q.dtype) if tol is None else tol, log=say)
    t = attn_tol(q.dtype) if tol is None else tol
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    assert err <= t, f"{what}: max abs err {err:.3e} > {t}"
    return err / t


# ------------------------------------------------------------------------------------------
# runners
# ------------------------------------------------------------------------------------------

def run_meta(qs, wl, sentinel=7.0):
    shape = (wl.num_meta_blocks, wl.BS, wl.N, wl.D)
    mx = torch.full(shape, sentinel, dtype=wl.k_cache.dtype, device=DEV)
    mn = torch.full(shape, sentinel, dtype=wl.k_cache.dtype, device=DEV)
    qs.qs_build_metadata(wl.k_cache.to(DEV), wl.block_tables.to(DEV), wl.meta_seq_lens.to(DEV),
                         wl.meta_tables.to(DEV), mx, mn)
    return mx, mn


def oracle_meta(oracle, wl, sentinel=7.0):
    shape = (wl.num_meta_blocks, wl.BS, wl.N, wl.D)
    s = torch.full(shape, sentinel, dtype=wl.k_cache.dtype)
    return oracle.build_metadata(wl.k_cache.cpu(), wl.block_tables.cpu(), wl.meta_seq_lens.cpu(),
                                 wl.meta_tables.cpu(), wl.num_meta_blocks, maxb=s, minb=s)


def run_select(qs, wl, mx, mn, k=None, scores=True):
    k = k or wl.k
    B, N = wl.B, wl.N
    sc = torch.full((B, N, wl.mmbpr * wl.BS), float("inf"), device=DEV) if scores else None
    ts = None if wl.tsmu is None else wl.tsmu.to(DEV)
    sel, ns = qs.qs_block_select(wl.query.to(DEV), mx, mn, wl.meta_tables.to(DEV), wl.seq_lens.to(DEV), k,
                                 tokens_since_update=ts, flags=wl.flags, block_scores=sc)
    return sel, ns, sc


def nbs_of(wl):
    return [cdiv(max(int(x), 0), wl.BS) for x in wl.seq_lens.cpu().tolist()]


# ------------------------------------------------------------------------------------------
# metadata
# ------------------------------------------------------------------------------------------

META_CASES = [
    # seed, B, N, BS, lens, dtype
    (1, 3, 8, 128, [128 * 5 + 3, 1, 128], torch.bfloat16),
    (2, 4, 2, 32, [0, 31, 32 * 33 + 7, 32 * 64], torch.float32),
    (3, 2, 1, 16, [16 * 16 * 2 + 1, 5], torch.bfloat16),
    (4, 2, 4, 64, [64 * 70, 64 * 3 - 1], torch.float32),
    (5, 1, 16, 128, [128 * 3 + 100], torch.bfloat16),
    (6, 2, 4, 64, [64 * 20 + 5, 64 * 3], torch.float16),
]


@pytest.mark.parametrize("case", META_CASES, ids=lambda c: f"seed{c[0]}")
def test_metadata_random(qs, oracle, case):
    seed, B, N, BS, lens, dtype = case
    say(f"metadata random seed={seed} B={B} N={N} BS={BS} dtype={dtype}")
    wl = W.random_case(seed, B, 2 * N, N, BS, lens, k=4, dtype=dtype, with_v=False)
    mx, mn = run_meta(qs, wl)
    torch.cuda.synchronize()
    omx, omn = oracle_meta(oracle, wl)
    assert np.array_equal(bits(tnp(mx)), bits(omx))
    assert np.array_equal(bits(tnp(mn)), bits(omn))


def test_metadata_signed_zeros(qs, oracle):
    say("metadata signed zeros")
    wl = W.random_case(6, 1, 2, 1, 32, [64], k=2, dtype=torch.bfloat16, with_v=False)
    kc = wl.k_cache.clone()
    kc[:, :, 0, :8] = 0.0
    kc[:, 5, 0, :4] = -0.0
    kc[:, :, 0, 8:16] = -0.0
    kc[:, 9, 0, 8:12] = 0.0
    wl.k_cache = kc
    mx, mn = run_meta(qs, wl)
    omx, omn = oracle_meta(oracle, wl)
    assert np.array_equal(bits(tnp(mx)), bits(omx)) and np.array_equal(bits(tnp(mn)), bits(omn))


def test_metadata_tiny_and_page3_example(qs, oracle):
    wl = W.tiny_needle()
    say("metadata, tiny workload")
    mx, mn = run_meta(qs, wl)
    omx, omn = oracle_meta(oracle, wl)
    assert np.array_equal(bits(tnp(mx)), bits(omx)) and np.array_equal(bits(tnp(mn)), bits(omn))
    say("metadata, page-3 example (full size, 640 MiB K cache)")
    wl = W.page3_select(device=DEV)
    mx, mn = run_meta(qs, wl)
    omx, omn = oracle_meta(oracle, wl)
    assert np.array_equal(bits(tnp(mx)), bits(omx)) and np.array_equal(bits(tnp(mn)), bits(omn))


# metadata refresh of the newest blocks
UPDATE_CASES = [
    # seed, B, N, BS, lens, first_block, max_new, dtype   (column slices per block in brackets)
    (21, 2, 8, 128, [128 * 9 + 3, 128 * 4], [8, 2], 1, torch.bfloat16),                 # [8]
    (22, 4, 2, 32, [0, 31, 32 * 33 + 7, 32 * 64], [0, -5, 30, 63], 4, torch.float32),   # [4]
    (23, 3, 3, 16, [16 * 16 * 2 + 1, 5, 16 * 20], [31, 0, 14], 3, torch.bfloat16),       # N=3: [2]
    (24, 2, 4, 64, [64 * 70, 64 * 3 - 1], [60, 1], 16, torch.float32),                   # [4]
    (25, 3, 1, 128, [128 * 3 + 100, 128 * 2, 1], [1, 5, 0], 2, torch.bfloat16),          # N=1: [1]
    (26, 8, 8, 16, [16 * 16 * 4] * 8, [0] * 8, 256, torch.bfloat16),                     # whole sequences: [1]
    (28, 2, 4, 32, [32 * 40 + 9, 32 * 7], [39, 3], 2, torch.float16),                    # [4]
]


@pytest.mark.parametrize("case", UPDATE_CASES, ids=lambda c: f"seed{c[0]}")
def test_update_metadata_random(qs, oracle, case):
    seed, B, N, BS, lens, first, max_new, dtype = case
    say(f"metadata refresh seed={seed} B={B} N={N} BS={BS} first={first} max_new={max_new} dtype={dtype}")
    wl = W.random_case(seed, B, 2 * N, N, BS, lens, k=4, dtype=dtype, with_v=False)
    shape = (wl.num_meta_blocks, BS, N, wl.D)
    mx = torch.full(shape, 7.0, dtype=dtype, device=DEV)
    mn = torch.full(shape, 7.0, dtype=dtype, device=DEV)
    fb = torch.tensor(first, dtype=torch.int32)
    qs.qs_update_metadata(wl.k_cache.to(DEV), wl.block_tables.to(DEV), wl.seq_lens.to(DEV), fb.to(DEV), max_new,
                          wl.meta_tables.to(DEV), mx, mn)
    torch.cuda.synchronize()
    s = torch.full(shape, 7.0, dtype=dtype)
    omx, omn = oracle.update_metadata(wl.k_cache, wl.block_tables, wl.seq_lens, fb, max_new, wl.meta_tables, s, s)
    assert np.array_equal(bits(tnp(mx)), bits(omx))
    assert np.array_equal(bits(tnp(mn)), bits(omn))


def test_update_metadata_serving_chain(qs, oracle):
    """Build after prefill, then a refresh every BS decoded tokens (from the block that was
    partial at the last refresh), on a zero-filled pool: the GPU pool equals the oracle's
    full build at the final length, bit for bit."""
    BS, N = 32, 8
    L0 = [32 * 50 + 9, 32 * 3, 1, 32 * 31]
    steps = 3 * BS + 11
    final = [x + steps for x in L0]
    say(f"metadata refresh chain BS={BS} L0={L0} steps={steps}")
    wl = W.random_case(27, len(L0), 16, N, BS, final, k=4, dtype=torch.bfloat16, with_v=False)
    kc, bt, mt = wl.k_cache.to(DEV), wl.block_tables.to(DEV), wl.meta_tables.to(DEV)
    mx = torch.zeros((wl.num_meta_blocks, BS, N, wl.D), dtype=torch.bfloat16, device=DEV)
    mn = torch.zeros_like(mx)
    cur = list(L0)
    qs.qs_build_metadata(kc, bt, torch.tensor(cur, dtype=torch.int32, device=DEV), mt, mx, mn)
    while cur != final:
        new = [min(x + BS, f) for x, f in zip(cur, final)]
        fb = torch.tensor([x // BS for x in cur], dtype=torch.int32, device=DEV)
        qs.qs_update_metadata(kc, bt, torch.tensor(new, dtype=torch.int32, device=DEV), fb, 2, mt, mx, mn)
        cur = new
    torch.cuda.synchronize()
    z = torch.zeros((wl.num_meta_blocks, BS, N, wl.D), dtype=torch.bfloat16)
    omx, omn = oracle.build_metadata(wl.k_cache, wl.block_tables, wl.seq_lens, wl.meta_tables, wl.num_meta_blocks,
                                     maxb=z, minb=z)
    assert np.array_equal(bits(tnp(mx)), bits(omx)) and np.array_equal(bits(tnp(mn)), bits(omn))


def test_decode_loop_refresh_select_attend(qs, oracle):
    """Page 3's serving loop on a small paged batch: metadata built after the prefill; each
    decode step appends one token per request (the pools already hold it; the length
    grows), runs the fused Quest selection + attention with per-request tokens_since_update
    and sink + window forcing, and every BS tokens since its last refresh a request has its
    newest blocks refreshed (from the block that was partial then). Every step's selection
    equals the oracle's over metadata the oracle builds for the covered tokens (up to near
    ties), and every output the oracle's attention over the GPU's selection."""
    BS, N, H, k = 16, 2, 8, 6
    L0 = [16 * 20 + 5, 16 * 7, 33]
    steps = 2 * BS + 7
    final = [x + steps for x in L0]
    B = len(L0)
    say(f"decode loop BS={BS} L0={L0} steps={steps}")
    wl = W.random_case(31, B, H, N, BS, final, k=k, dtype=torch.float32)
    kc, vc, bt, mt = (t.to(DEV) for t in (wl.k_cache, wl.v_cache, wl.block_tables, wl.meta_tables))
    shape = (wl.num_meta_blocks, BS, N, wl.D)
    mx = torch.zeros(shape, device=DEV)
    mn = torch.zeros(shape, device=DEV)
    cur, covered = list(L0), list(L0)
    qs.qs_build_metadata(kc, bt, torch.tensor(cur, dtype=torch.int32, device=DEV), mt, mx, mn)
    flags = W.FORCE_SINK | W.FORCE_WINDOW
    gen = torch.Generator().manual_seed(31)
    for step in range(steps):
        cur = [x + 1 for x in cur]
        due = [c - cv >= BS for c, cv in zip(cur, covered)]
        if any(due):
            # requests not due get first_block = nb: nothing of theirs is written
            fb = [cv // BS if d else cdiv(c, BS) for c, cv, d in zip(cur, covered, due)]
            qs.qs_update_metadata(kc, bt, torch.tensor(cur, dtype=torch.int32, device=DEV),
                                  torch.tensor(fb, dtype=torch.int32, device=DEV), 2, mt, mx, mn)
            covered = [c if d else cv for c, cv, d in zip(cur, covered, due)]
        tsmu = [c - cv for c, cv in zip(cur, covered)]
        q = (torch.rand((B, H, wl.D), generator=gen) * 2 - 1).float()
        sl = torch.tensor(cur, dtype=torch.int32)
        ts = torch.tensor(tsmu, dtype=torch.int32)
        sel = torch.full((B, N, k), -7, dtype=torch.int32, device=DEV)
        ns = torch.full((B, N), -7, dtype=torch.int32, device=DEV)
        out = qs.qs_select_attn_decode(q.to(DEV), mx, mn, mt, kc, vc, bt, sl.to(DEV), k, tokens_since_update=ts.to(DEV),
                                       flags=flags, selected=sel, n_selected=ns)
        torch.cuda.synchronize()
        z = np.zeros(shape, dtype=np.float32)
        omx, omn = oracle.build_metadata(wl.k_cache, wl.block_tables, torch.tensor(covered, dtype=torch.int32),
                                         wl.meta_tables, wl.num_meta_blocks, maxb=z, minb=z)
        osel, ons, osc = oracle.block_select(q, omx, omn, wl.meta_tables, sl, k, tsmu=ts, flags=flags)
        compare_quest(tnp(sel), tnp(ns), osel, ons, osc, [cdiv(c, BS) for c in cur], k)
        ref = oracle.sparse_attn_decode(q, wl.k_cache, wl.v_cache, wl.block_tables, sl, tnp(sel), tnp(ns), N)
        err = float(np.abs(out.cpu().numpy() - ref).max())
        assert err <= 1e-4, f"step {step}: attention err {err:.3e}"
    assert covered != L0  # every request was refreshed at least once


def test_update_metadata_serving_newest_blocks(qs, oracle):
    """Serving shape (B=128, N=8, BS=128, 256 blocks a request, 8 GiB K pool): refresh the
    last blocks of every request in one call; every request against the oracle, and no
    row outside the refreshed blocks written anywhere in the pool."""
    wl = W.serving(device=DEV)
    first, max_new = 250, 8                 # blocks 250 .. 255 (nb = 256)
    say(f"metadata refresh, serving shape, first={first} max_new={max_new}")
    shape = (wl.num_meta_blocks, wl.BS, wl.N, wl.D)
    mx = torch.full(shape, 7.0, dtype=torch.bfloat16, device=DEV)
    mn = torch.full(shape, 7.0, dtype=torch.bfloat16, device=DEV)
    fb = torch.full((wl.B,), first, dtype=torch.int32, device=DEV)
    qs.qs_update_metadata(wl.k_cache, wl.block_tables, wl.meta_seq_lens, fb, max_new, wl.meta_tables, mx, mn)
    torch.cuda.synchronize()
    # rows of blocks 250..255 live in each request's second metadata block, rows 122..127
    nb = cdiv(int(wl.meta_seq_lens[0]), wl.BS)
    assert nb == 256 and bool((wl.meta_seq_lens == wl.meta_seq_lens[0]).all())
    sentinel = torch.tensor(7.0, dtype=torch.bfloat16)
    written = torch.zeros((wl.num_meta_blocks, wl.BS), dtype=torch.bool, device=DEV)
    mt = wl.meta_tables.cpu()
    for b in range(wl.B):
        written[int(mt[b, 1]), first - wl.BS:nb - wl.BS] = True
    for t in (mx, mn):
        is_sent = (t == sentinel.to(DEV)).flatten(2).all(dim=2)
        assert bool(is_sent[~written].all()), "a row outside the refreshed blocks was written"
    gmx, gmn = bits(tnp(mx)), bits(tnp(mn))
    for c0 in range(0, wl.B, 32):                 # every request, 32 at a time
        reqs = list(range(c0, min(wl.B, c0 + 32)))
        sub, nbs = gather_requests(wl, reqs, with_v=False)
        s = torch.full((sub.num_meta_blocks, wl.BS, wl.N, wl.D), 7.0, dtype=torch.bfloat16)
        omx, omn = oracle.update_metadata(sub.k_cache, sub.block_tables, sub.meta_seq_lens,
                                          torch.full((len(reqs),), first, dtype=torch.int32), max_new,
                                          sub.meta_tables, s, s)
        bx, bn = bits(omx), bits(omn)
        for j, b in enumerate(reqs):
            for m in range(cdiv(nbs[j], wl.BS)):
                om = int(sub.meta_tables[j, m])
                assert np.array_equal(gmx[int(mt[b, m])], bx[om]) and np.array_equal(gmn[int(mt[b, m])], bn[om]), b


# ------------------------------------------------------------------------------------------
# Quest select
# ------------------------------------------------------------------------------------------

SELECT_CASES = [
    # seed, B, H, N, BS, lens, k, dtype, flags, tsmu
    (11, 3, 8, 2, 32, [32 * 40 + 5, 32 * 7, 1], 5, torch.float32, 0, None),
    (12, 4, 32, 8, 128, [128 * 300 + 17, 128 * 64, 0, 128 * 129], 8, torch.bfloat16, 0, None),
    (13, 2, 16, 8, 128, [128 * 200, 128 * 3], 16, torch.bfloat16, 3, [0, 0]),
    (14, 3, 16, 4, 64, [64 * 100 + 9, 64 * 20, 64 * 65], 12, torch.bfloat16, 3, [9, 200, -1]),
    (15, 2, 4, 1, 16, [16 * 16 * 3 + 2, 16 * 5], 40, torch.float32, 1, None),
    (16, 2, 8, 8, 32, [32 * 100, 32 * 2], 1, torch.float32, 2, [0, 64]),
    (17, 1, 64, 8, 128, [128 * 1024], 64, torch.bfloat16, 3, [127]),
    (18, 2, 24, 8, 64, [64 * 130 + 1, 64 * 66], 9, torch.bfloat16, 3, [1, 0]),
    (19, 3, 16, 4, 64, [64 * 90 + 3, 64 * 17, 64 * 200], 10, torch.float16, 3, [3, 0, 70]),
]


@pytest.mark.parametrize("case", SELECT_CASES, ids=lambda c: f"seed{c[0]}")
def test_block_select_random(qs, oracle, case):
    seed, B, H, N, BS, lens, k, dtype, flags, tsmu = case
    say(f"select random seed={seed} B={B} H={H} N={N} BS={BS} k={k} flags={flags}")
    cover = None if tsmu is None else [max(0, L - max(t, 0)) for L, t in zip(lens, tsmu)]
    wl = W.random_case(seed, B, H, N, BS, lens, k=k, dtype=dtype, with_v=False, meta_cover=cover,
                       tsmu=tsmu, flags=flags)
    mx, mn = run_meta(qs, wl, sentinel=0.0)
    sel, ns, sc = run_select(qs, wl, mx, mn, k)
    torch.cuda.synchronize()
    omx, omn = oracle_meta(oracle, wl, sentinel=0.0)
    osel, ons, osc = oracle.block_select(wl.query, omx, omn, wl.meta_tables, wl.seq_lens, k,
                                         tsmu=wl.tsmu, flags=flags)
    nbs = nbs_of(wl)
    gsc = tnp(sc)
    mask = np.zeros_like(osc, dtype=bool)
    for b, nb in enumerate(nbs):
        mask[b, :, :nb] = ~np.isnan(osc[b, :, :nb])
        forced = np.isnan(osc[b, :, :nb])
        assert np.all(np.isnan(gsc[b, :, :nb][forced])), "forced blocks must carry NaN scores"
    check_scores(gsc, osc, mask)
    compare_quest(tnp(sel), tnp(ns), osel, ons, osc, nbs, k)


def test_block_select_long_row_scores_in_global_memory(qs, oracle):
    """One request of 9001 blocks at BS=16: more candidates than the LDS score capacity, so
    the top-k kernel selects from the workspace scores; 563 metadata-table entries."""
    say("select long row (9001 blocks)")
    wl = W.random_case(19, 1, 4, 1, 16, [16 * 9000 + 7], k=100, dtype=torch.bfloat16, with_v=False,
                       tsmu=[5], flags=W.FORCE_SINK | W.FORCE_WINDOW)
    assert wl.mmbpr * wl.BS > 8192
    mx, mn = run_meta(qs, wl)
    sel, ns, sc = run_select(qs, wl, mx, mn)
    omx, omn = oracle_meta(oracle, wl)
    osel, ons, osc = oracle.block_select(wl.query, omx, omn, wl.meta_tables, wl.seq_lens, wl.k, tsmu=wl.tsmu,
                                         flags=wl.flags)
    nbs = nbs_of(wl)
    mask = np.zeros_like(osc, dtype=bool)
    mask[0, :, :nbs[0]] = ~np.isnan(osc[0, :, :nbs[0]])
    check_scores(tnp(sc), osc, mask)
    compare_quest(tnp(sel), tnp(ns), osel, ons, osc, nbs, wl.k)


def test_block_select_row_mode_with_wide_table(qs, oracle):
    """512 rows (row mode) with a 257-entry metadata table (too wide to stage in LDS, so the
    lookups go to global memory): one long request among short ones."""
    say("select row mode, 257 metadata blocks")
    lens = [16 * (256 * 16 + 1)] + [16 * (1 + b % 5) + b % 7 for b in range(63)]
    wl = W.random_case(20, 64, 8, 8, 16, lens, k=12, dtype=torch.bfloat16, with_v=False)
    assert wl.mmbpr == 257 and wl.B * wl.N >= 512
    mx, mn = run_meta(qs, wl)
    sel, ns, sc = run_select(qs, wl, mx, mn)
    omx, omn = oracle_meta(oracle, wl)
    osel, ons, osc = oracle.block_select(wl.query, omx, omn, wl.meta_tables, wl.seq_lens, wl.k)
    compare_quest(tnp(sel), tnp(ns), osel, ons, osc, nbs_of(wl), wl.k)


def test_block_select_exact_ties(qs, oracle):
    """Metadata with few distinct values: many exactly equal scores; the lower index
    must win every tie (the oracle and the GPU then agree exactly)."""
    say("select exact ties")
    B, H, N, BS, D = 2, 8, 2, 32, 128
    g = torch.Generator().manual_seed(7)
    nmeta = 4
    mx = torch.randint(-1, 2, (nmeta, BS, N, D), generator=g).float()
    mn = mx - torch.randint(0, 2, (nmeta, BS, N, D), generator=g).float()
    q = torch.ones((B, H, D))
    mt = torch.tensor([[0, 1], [2, 3]], dtype=torch.int32)
    sl = torch.tensor([BS * 60, BS * 33 + 1], dtype=torch.int32)
    for k in (1, 7, 32):
        sel, ns = qs.qs_block_select(q.to(DEV), mx.to(DEV), mn.to(DEV), mt.to(DEV), sl.to(DEV), k)
        osel, ons, _ = oracle.block_select(q, mx, mn, mt, sl, k)
        np.testing.assert_array_equal(tnp(sel), osel)
        np.testing.assert_array_equal(tnp(ns), ons)


def test_block_select_topk_uniform_and_clustered(qs, oracle):
    """Score distributions that reach every branch of the exact top-k: all candidates equal
    (only the index order decides), and one outlier above a tight cluster with repeated
    values, where far more than 256 candidates share the histogram bin of the k-th best
    score. A one-hot query makes each block's score exactly its channel-0 metadata value,
    so the GPU (fp32) and the oracle (fp64) see identical scores and must agree exactly."""
    BS, D, nb = 32, 128, 2000
    nmeta = cdiv(nb, BS)
    q = torch.zeros((1, 1, D))
    q[0, 0, 0] = 1.0
    mt = torch.arange(nmeta, dtype=torch.int32)[None]
    sl = torch.tensor([nb * BS], dtype=torch.int32)
    j = torch.arange(nb)
    uniform = torch.zeros(nb)
    clustered = 1.0 + ((j * 37) % 500).float() * 2.0 ** -20   # each value on 4 blocks
    clustered[0] = 1.0e4
    for name, v in (("uniform", uniform), ("clustered", clustered)):
        mx = torch.zeros((nmeta * BS, 1, D))
        mx[:nb, 0, 0] = v
        mx = mx.reshape(nmeta, BS, 1, D)
        for k in (1, 2, 10, 300):
            say(f"select top-k {name} k={k}")
            sel, ns = qs.qs_block_select(q.to(DEV), mx.to(DEV), mx.to(DEV), mt.to(DEV), sl.to(DEV), k)
            osel, ons, _ = oracle.block_select(q, mx, mx, mt, sl, k)
            np.testing.assert_array_equal(tnp(sel), osel)
            np.testing.assert_array_equal(tnp(ns), ons)


def test_block_select_tiny_needle(qs, oracle):
    say("select, tiny workload")
    wl = W.tiny_needle()
    mx, mn = run_meta(qs, wl)
    sel, ns, sc = run_select(qs, wl, mx, mn)
    omx, omn = oracle_meta(oracle, wl)
    osel, ons, osc = oracle.block_select(wl.query, omx, omn, wl.meta_tables, wl.seq_lens, wl.k)
    compare_quest(tnp(sel), tnp(ns), osel, ons, osc, nbs_of(wl), wl.k)
    needle_block = wl.needles[0][1] // wl.BS
    assert needle_block in set(tnp(sel)[0, 0].tolist())


@pytest.mark.parametrize("flags", [0, W.FORCE_SINK | W.FORCE_WINDOW])
def test_block_select_page3_example_full(qs, oracle, flags):
    say(f"select, page-3 example, full size, flags={flags}")
    wl = W.page3_select(device=DEV)
    wl.flags = flags
    if flags:
        wl.tsmu = torch.zeros(wl.B, dtype=torch.int32, device=DEV)
    mx, mn = run_meta(qs, wl)
    sel, ns, sc = run_select(qs, wl, mx, mn)
    omx, omn = oracle_meta(oracle, wl)
    osel, ons, osc = oracle.block_select(wl.query.cpu(), omx, omn, wl.meta_tables.cpu(), wl.seq_lens.cpu(),
                                         wl.k, tsmu=None if wl.tsmu is None else wl.tsmu.cpu(), flags=flags)
    nbs = nbs_of(wl)
    check_scores(tnp(sc), osc, ~np.isnan(osc) & (np.arange(osc.shape[2]) < 128)[None, None, :])
    compare_quest(tnp(sel), tnp(ns), osel, ons, osc, nbs, wl.k)


def test_block_select_deterministic(qs):
    say("select determinism")
    wl = W.random_case(19, 4, 32, 8, 128, [128 * 500, 128 * 77 + 3, 128 * 1000, 128 * 2], k=16,
                       dtype=torch.bfloat16, with_v=False)
    mx, mn = run_meta(qs, wl)
    outs = [run_select(qs, wl, mx, mn) for _ in range(3)]
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b)


# ------------------------------------------------------------------------------------------
# probe select
# ------------------------------------------------------------------------------------------

PROBE_CASES = [
    # seed, B, H, N, BS, lens, k, dtype, importance, flags, n_probe
    (21, 2, 4, 2, 32, [32 * 40 + 20, 32 * 9], 6, torch.float32, True, 4, 8),
    (22, 2, 16, 8, 32, [32 * 128, 32 * 3 + 1], 32, torch.float32, True, 4, 8),
    (23, 1, 8, 8, 64, [64 * 50 + 3], 5, torch.bfloat16, False, 4, 8),
    (24, 3, 4, 4, 16, [16 * 30, 0, 16 * 7 + 5], 9, torch.float32, True, 0, 3),
    (25, 1, 4, 2, 32, [32 * 70], 4, torch.bfloat16, True, 4, 64),
    (26, 1, 2, 1, 128, [128 * 40 + 77], 3, torch.float32, True, 4, 0),
    (27, 2, 8, 4, 32, [32 * 60 + 9, 32 * 5], 7, torch.float16, True, 4, 8),
]


@pytest.mark.parametrize("case", PROBE_CASES, ids=lambda c: f"seed{c[0]}")
def test_probe_select_random(qs, oracle, case):
    seed, B, H, N, BS, lens, k, dtype, use_imp, flags, n_probe = case
    say(f"probe random seed={seed} B={B} H={H} N={N} BS={BS} k={k} imp={use_imp} flags={flags} n_probe={n_probe}")
    wl = W.random_case(seed, B, H, N, BS, lens, k=k, dtype=dtype, with_v=False, with_importance=use_imp)
    imp = wl.importance if use_imp else None
    ps = torch.full((B, H, wl.mkbpr), float("inf"), device=DEV)
    sel, ns = qs.qs_probe_select(wl.query.to(DEV), wl.k_cache.to(DEV), wl.block_tables.to(DEV),
                                 wl.seq_lens.to(DEV), k, importance=None if imp is None else imp.to(DEV),
                                 n_probe=n_probe, flags=flags, probe_scores=ps)
    o = oracle.probe_select(wl.query, wl.k_cache, wl.block_tables, wl.seq_lens, k, N, importance=imp,
                            n_probe=n_probe, flags=flags)
    nbs = nbs_of(wl)
    mask = np.zeros(o["probe"].shape, dtype=bool)
    for b, nb in enumerate(nbs):
        mask[b, :, :nb] = True
    check_scores(tnp(ps), o["probe"], mask)
    compare_probe(tnp(sel), tnp(ns), o, nbs, k)


def test_probe_select_at_block_capacity(qs, oracle):
    """The probe selection's largest row: 4096 blocks (BS=16, 65536 tokens), with importance,
    recency and k=200."""
    say("probe select at 4096 blocks")
    wl = W.random_case(28, 1, 2, 1, 16, [16 * 4096], k=200, dtype=torch.float32, with_v=False,
                       with_importance=True)
    assert wl.mkbpr == 4096
    ps = torch.full((1, 2, 4096), float("inf"), device=DEV)
    sel, ns = qs.qs_probe_select(wl.query.to(DEV), wl.k_cache.to(DEV), wl.block_tables.to(DEV), wl.seq_lens.to(DEV),
                                 200, importance=wl.importance.to(DEV), n_probe=8, flags=W.RECENCY,
                                 probe_scores=ps)
    o = oracle.probe_select(wl.query, wl.k_cache, wl.block_tables, wl.seq_lens, 200, 1, importance=wl.importance,
                            n_probe=8, flags=W.RECENCY)
    check_scores(tnp(ps), o["probe"], np.ones(o["probe"].shape, dtype=bool))
    compare_probe(tnp(sel), tnp(ns), o, nbs_of(wl), 200)


def test_probe_select_page1_k_sweep(qs, oracle):
    wl = W.page1_probe()
    for k in (1, 2, 4, 8, 16, 32):
        say(f"probe, page-1 workload, k={k}")
        sel, ns = qs.qs_probe_select(wl.query.to(DEV), wl.k_cache.to(DEV), wl.block_tables.to(DEV),
                                     wl.seq_lens.to(DEV), k, importance=wl.importance.to(DEV), n_probe=8,
                                     flags=W.RECENCY)
        o = oracle.probe_select(wl.query, wl.k_cache, wl.block_tables, wl.seq_lens, k, wl.N,
                                importance=wl.importance, n_probe=8, flags=W.RECENCY)
        compare_probe(tnp(sel), tnp(ns), o, nbs_of(wl), k)
        if k == 1:
            best = int(np.argmax(o["imp_sum"][0, :128]))
            assert np.all(tnp(sel)[0, :, 0] == best)


# ------------------------------------------------------------------------------------------
# sparse attention
# ------------------------------------------------------------------------------------------

def random_selection(seed, B, rows, k, nbs, extra_invalid=True):
    g = torch.Generator().manual_seed(seed)
    sel = torch.full((B, rows, k), -1, dtype=torch.int32)
    ns = torch.zeros((B, rows), dtype=torch.int32)
    for b in range(B):
        nb = nbs[b]
        for r in range(rows):
            m = min(k, nb)
            if m == 0:
                continue
            pick = torch.randperm(nb, generator=g)[:m].sort().values.to(torch.int32)
            sel[b, r, :m] = pick
            ns[b, r] = m
            if extra_invalid and r % 3 == 1 and m < k:
                sel[b, r, m] = nb + 5        # out of range: skipped
                ns[b, r] = m + 1
    return sel, ns


ATTN_CASES = [
    # seed, B, H, N, BS, lens, k, kv dtype, q dtype, sel_heads factor (1 -> N, 0 -> H)
    (31, 2, 8, 2, 32, [32 * 20 + 7, 32 * 3], 6, torch.float32, torch.float32, 1),
    (32, 3, 32, 8, 128, [128 * 70 + 1, 128 * 16, 0], 16, torch.bfloat16, torch.bfloat16, 1),
    (33, 2, 64, 8, 128, [128 * 40, 128 * 33 + 64], 16, torch.bfloat16, torch.bfloat16, 1),
    (34, 1, 16, 8, 32, [32 * 128], 32, torch.float32, torch.float32, 0),
    (35, 2, 16, 8, 32, [32 * 100 + 3, 32 * 50], 12, torch.int8, torch.float32, 0),
    (36, 2, 32, 8, 64, [64 * 30 + 11, 64 * 8], 7, torch.int8, torch.bfloat16, 1),
    (37, 1, 24, 8, 64, [64 * 20], 5, torch.bfloat16, torch.bfloat16, 1),       # 3 heads per row
    (38, 1, 40, 2, 16, [16 * 50 + 1], 9, torch.float32, torch.float32, 1),     # 20 heads per row
    (39, 4, 4, 1, 128, [128 * 64, 1, 128 * 2, 0], 64, torch.bfloat16, torch.bfloat16, 1),
    (40, 1, 8, 8, 16, [16 * 8], 1, torch.float32, torch.float32, 1),
    (42, 2, 32, 8, 128, [128 * 40 + 5, 128 * 9], 12, torch.float16, torch.float16, 1),   # f16 matrix cores
    (43, 2, 16, 8, 32, [32 * 50 + 1, 32 * 7], 9, torch.float16, torch.float32, 0),       # f16 KV, fp32 query
    (44, 2, 8, 2, 32, [32 * 30, 32 * 4 + 2], 5, torch.float32, torch.float16, 1),        # fp32 KV, f16 query
    # 512 rows -> 2 splits of 100 slots: longer than one wave's slot table (lookups in the loop)
    (45, 8, 64, 8, 16, [16 * 210 + (7 * b) % 16 for b in range(8)], 200, torch.bfloat16, torch.bfloat16, 0),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: f"seed{c[0]}")
def test_sparse_attn_random(qs, oracle, case):
    seed, B, H, N, BS, lens, k, kvd, qd, shf = case
    say(f"attn random seed={seed} B={B} H={H} N={N} BS={BS} k={k} kv={kvd} q={qd}")
    int8 = kvd == torch.int8
    wl = W.random_case(seed, B, H, N, BS, lens, k=k, dtype=torch.float32 if int8 else kvd, int8=int8)
    q = wl.query.to(qd)
    kc, vc = (wl.k_i8, wl.v_i8) if int8 else (wl.k_cache, wl.v_cache)
    sel_heads = N if shf == 1 else H
    sel, ns = random_selection(seed, B, sel_heads, k, nbs_of(wl))
    out = qs.qs_sparse_attn_decode(q.to(DEV), kc.to(DEV), vc.to(DEV), wl.block_tables.to(DEV),
                                   wl.seq_lens.to(DEV), sel.to(DEV), ns.to(DEV), sel_heads=sel_heads,
                                   k_scale=None if not int8 else wl.k_scale.to(DEV),
                                   v_scale=None if not int8 else wl.v_scale.to(DEV))
    ref = oracle.sparse_attn_decode(q, kc, vc, wl.block_tables, wl.seq_lens, sel, ns, sel_heads,
                                    k_scale=wl.k_scale if int8 else None, v_scale=wl.v_scale if int8 else None)
    check_attn(out, ref, q, kc, vc, wl.block_tables, wl.seq_lens, sel, ns, sel_heads, f"attn seed={seed}",
               tol=2e-5 if int8 and qd == torch.float32 else None)


def test_sparse_attn_empty_rows_write_zeros(qs):
    say("attn empty selections")
    wl = W.random_case(41, 2, 8, 2, 32, [0, 32 * 4], k=3)
    sel = torch.full((2, 2, 3), -1, dtype=torch.int32)
    ns = torch.tensor([[0, 3], [0, 2]], dtype=torch.int32)
    out = torch.full((2, 8, 128), 5.0, device=DEV)
    qs.qs_sparse_attn_decode(wl.query.to(DEV), wl.k_cache.to(DEV), wl.v_cache.to(DEV), wl.block_tables.to(DEV),
                             wl.seq_lens.to(DEV), sel.to(DEV), ns.to(DEV), out=out)
    assert torch.all(out == 0)


def test_sparse_attn_tiny(qs, oracle):
    say("attn, tiny workload (oracle selection)")
    wl = W.tiny_needle()
    omx, omn = oracle_meta(oracle, wl)
    osel, ons, _ = oracle.block_select(wl.query, omx, omn, wl.meta_tables, wl.seq_lens, wl.k)
    out = qs.qs_sparse_attn_decode(wl.query.to(DEV), wl.k_cache.to(DEV), wl.v_cache.to(DEV),
                                   wl.block_tables.to(DEV), wl.seq_lens.to(DEV), torch.from_numpy(osel).to(DEV),
                                   torch.from_numpy(ons).to(DEV))
    ref = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, osel, ons, wl.N)
    assert np.abs(out.cpu().numpy() - ref).max() <= 1e-4


@pytest.mark.parametrize("int8", [False, True])
def test_sparse_attn_page1_probe(qs, oracle, int8):
    wl = W.page1_probe()
    kc, vc = (wl.k_i8, wl.v_i8) if int8 else (wl.k_cache, wl.v_cache)
    for k in (1, 2, 4, 8, 16, 32):
        say(f"attn, page-1 workload, k={k} int8={int8}")
        o = oracle.probe_select(wl.query, wl.k_cache, wl.block_tables, wl.seq_lens, k, wl.N,
                                importance=wl.importance, n_probe=8, flags=W.RECENCY)
        sel, ns = torch.from_numpy(o["selected"]), torch.from_numpy(o["n_selected"])
        out = qs.qs_sparse_attn_decode(wl.query.to(DEV), kc.to(DEV), vc.to(DEV), wl.block_tables.to(DEV),
                                       wl.seq_lens.to(DEV), sel.to(DEV), ns.to(DEV), sel_heads=wl.H,
                                       k_scale=wl.k_scale.to(DEV) if int8 else None,
                                       v_scale=wl.v_scale.to(DEV) if int8 else None)
        ref = oracle.sparse_attn_decode(wl.query, kc, vc, wl.block_tables, wl.seq_lens, sel, ns, wl.H,
                                        k_scale=wl.k_scale if int8 else None, v_scale=wl.v_scale if int8 else None)
        err = np.abs(out.cpu().numpy() - ref).max()
        assert err <= (2e-5 if int8 else 1e-4), f"k={k} err {err:.3e}"


# ------------------------------------------------------------------------------------------
# fused selection + attention (qs_select_attn_decode)
# ------------------------------------------------------------------------------------------

FUSED_CASES = [
    # seed, B, H, N, BS, lens, k, dtype, flags, tsmu          path taken
    (71, 2, 8, 2, 32, [32 * 40 + 5, 32 * 7], 5, torch.float32, 0, None),         # one kernel, slot splits
    (72, 3, 32, 8, 128, [128 * 200 + 17, 128 * 64, 0], 8, torch.bfloat16, 3, [5, 0, 0]),   # one kernel, splits
    (73, 2, 40, 2, 64, [64 * 100 + 9, 64 * 3], 12, torch.bfloat16, 3, [9, -1]),  # G=20: two head chunks
    (74, 2, 40, 2, 16, [16 * 200 + 1, 16 * 20], 7, torch.float32, 1, None),       # fp32 G=20: three chunks
    (75, 2, 16, 8, 128, [128 * 600, 128 * 300 + 3], 64, torch.bfloat16, 3, [127, 0]),  # long rows: prescored
    (79, 3, 8, 2, 32, [32 * 400 + 5, 32 * 90, 1], 20, torch.float32, 3, [4, 0, 0]),   # fp32 prescored
    (76, 1, 8, 8, 32, [32 * 64], 65, torch.bfloat16, 0, None),                    # k > 64: two kernels
    (77, 128, 16, 8, 16, [16 * (20 + (7 * b) % 23) + b % 5 for b in range(128)], 6, torch.bfloat16, 3,
     [b % 16 for b in range(128)]),                                               # 1024 rows: one kernel, no split
    (78, 2, 32, 8, 128, [128 * 150 + 3, 128 * 20], 8, torch.float16, 3, [2, 0]),  # f16, one kernel, splits
    (80, 3, 8, 2, 16, [16 * 3 + 1, 1, 0], 9, torch.float32, 3, [0, 0, 0]),       # k > nb, 1 token, empty
    (81, 3, 16, 8, 64, [64 * 300 + 1, 64 * 2, 0], 64, torch.bfloat16, 3, [0, 0, 0]),  # prescored, k > nb, empty
    (82, 1, 8, 2, 16, [16 * 4096], 64, torch.bfloat16, 3, [3]),   # at the LDS capacity: 4096 blocks, 256 table entries
    (83, 1, 8, 2, 16, [16 * 4097 + 5], 64, torch.bfloat16, 3, [0]),  # one block past it: two kernels
]


def run_fused(qs, wl, mx, mn, want_sel=True):
    B, N, k = wl.B, wl.N, wl.k
    sel = torch.full((B, N, k), -7, dtype=torch.int32, device=DEV) if want_sel else None
    ns = torch.full((B, N), -7, dtype=torch.int32, device=DEV) if want_sel else None
    ts = None if wl.tsmu is None else wl.tsmu.to(DEV)
    out = qs.qs_select_attn_decode(wl.query.to(DEV), mx, mn, wl.meta_tables.to(DEV), wl.k_cache.to(DEV),
                                   wl.v_cache.to(DEV), wl.block_tables.to(DEV), wl.seq_lens.to(DEV), k,
                                   tokens_since_update=ts, flags=wl.flags, selected=sel, n_selected=ns)
    return out, sel, ns


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_pool_placement_does_not_change_results(qs, dtype):
    """K / V and max / min pools from the placement helpers (second pool 256 B past a 1 KiB
    multiple) against separately allocated ones: metadata, selection, fused and separate
    attention all bitwise equal."""
    say(f"pool placement dtype={dtype}")
    wl = W.random_case(115, 3, 16, 4, 64, [64 * 150 + 7, 64 * 9, 1], k=12, dtype=dtype, flags=3, tsmu=[3, 0, 0])
    q, bt, sl, mt = (t.to(DEV) for t in (wl.query, wl.block_tables, wl.seq_lens, wl.meta_tables))
    ts = wl.tsmu.to(DEV)
    kc, vc = wl.k_cache.to(DEV), wl.v_cache.to(DEV)
    kp, vp = qs.alloc_kv_pools(kc.shape[0], wl.BS, wl.N, wl.D, dtype=dtype, device=DEV)
    kp.copy_(kc)
    vp.copy_(vc)
    assert (vp.data_ptr() - kp.data_ptr()) % 1024 == 256
    outs = []
    for (k_, v_), paired in (((kc, vc), False), ((kp, vp), True)):
        if paired:
            mx, mn = qs.alloc_metadata_pools(wl.num_meta_blocks, wl.BS, wl.N, wl.D, dtype=dtype, device=DEV)
            assert (mn.data_ptr() - mx.data_ptr()) % 1024 == 256
        else:
            mx = torch.zeros((wl.num_meta_blocks, wl.BS, wl.N, wl.D), dtype=dtype, device=DEV)
            mn = torch.zeros_like(mx)
        qs.qs_build_metadata(k_, bt, sl, mt, mx, mn)
        sel, ns = qs.qs_block_select(q, mx, mn, mt, sl, wl.k, tokens_since_update=ts, flags=wl.flags)
        att = qs.qs_sparse_attn_decode(q, k_, v_, bt, sl, sel, ns)
        fused = qs.qs_select_attn_decode(q, mx, mn, mt, k_, v_, bt, sl, wl.k, tokens_since_update=ts, flags=wl.flags)
        torch.cuda.synchronize()
        outs.append([x.cpu() for x in (mx, mn, sel, ns, att, fused)])
    ib = torch.int32 if dtype == torch.float32 else torch.int16
    for a, b in zip(*outs):
        if a.is_floating_point():
            assert torch.equal(a.view(ib), b.view(ib))
        else:
            assert torch.equal(a, b)


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: f"seed{c[0]}")
def test_select_attn_random(qs, oracle, case):
    seed, B, H, N, BS, lens, k, dtype, flags, tsmu = case
    say(f"select+attention seed={seed} B={B} H={H} N={N} BS={BS} k={k} dtype={dtype} flags={flags}")
    wl = W.random_case(seed, B, H, N, BS, lens, k=k, dtype=dtype, tsmu=tsmu, flags=flags)
    mx, mn = run_meta(qs, wl, sentinel=0.0)
    out, sel, ns = run_fused(qs, wl, mx, mn)
    out2, _, _ = run_fused(qs, wl, mx, mn, want_sel=False)
    torch.cuda.synchronize()
    # the output does not depend on whether the selection is also written out
    ib = torch.int32 if dtype == torch.float32 else torch.int16
    assert torch.equal(out.view(ib), out2.view(ib))
    omx, omn = oracle_meta(oracle, wl, sentinel=0.0)
    osel, ons, osc = oracle.block_select(wl.query, omx, omn, wl.meta_tables, wl.seq_lens, k, tsmu=wl.tsmu,
                                         flags=wl.flags)
    gsel, gns = tnp(sel), tnp(ns)
    compare_quest(gsel, gns, osel, ons, osc, nbs_of(wl), k)
    ref = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, gsel, gns, N)
    check_attn(out, ref, wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, gsel, gns, N,
               f"select+attention seed={seed}")
    # consistency with the separate operations: the same selection, bit for bit
    s2, n2, _ = run_select(qs, wl, mx, mn, k=k, scores=False)
    assert np.array_equal(tnp(s2), gsel) and np.array_equal(tnp(n2), gns)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_select_attn_prescored_rows_with_exact_ties(qs, oracle, dtype):
    """Long rows selected per wave after the scoring grid (rows of 300-700 blocks): many
    blocks hold identical keys (copies of four blocks), so the k-th score is tied across
    many blocks and the lower indices must win. The fused selection is bitwise
    qs_block_select's and equals the oracle's exactly (ties broken by index); outputs
    match the oracle's attention."""
    lens = [64 * 500 + 3, 64 * 300, 64 * 700, 64 * 2 + 5]
    say(f"select+attention, prescored rows with exact ties, {dtype}")
    wl = W.random_case(85, 4, 32, 8, 64, lens, k=64, dtype=dtype, flags=W.FORCE_SINK | W.FORCE_WINDOW,
                       tsmu=[7, 0, 63, 1])
    wl.meta_seq_lens = wl.seq_lens - wl.tsmu
    src = wl.block_tables[0, :4].long()
    for b in range(3):
        nb = cdiv(lens[b], 64)
        for i in range(1, nb - 1):
            if i % 3:                                     # two of every three blocks copy one of four
                wl.k_cache[int(wl.block_tables[b, i])] = wl.k_cache[int(src[i % 4])]
    mx, mn = run_meta(qs, wl, sentinel=0.0)
    out, sel, ns = run_fused(qs, wl, mx, mn)
    s2, n2, _ = run_select(qs, wl, mx, mn, scores=False)
    torch.cuda.synchronize()
    assert torch.equal(sel, s2) and torch.equal(ns, n2)
    omx, omn = oracle_meta(oracle, wl, sentinel=0.0)
    osel, ons, osc = oracle.block_select(wl.query, omx, omn, wl.meta_tables, wl.seq_lens, wl.k, tsmu=wl.tsmu,
                                         flags=wl.flags)
    gsel, gns = tnp(sel), tnp(ns)
    compare_quest(gsel, gns, osel, ons, osc, nbs_of(wl), wl.k)
    ref = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, gsel, gns,
                                    wl.N)
    check_attn(out, ref, wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, gsel, gns, wl.N,
               "prescored rows with ties")


def test_select_attn_tiny(qs, oracle):
    wl = W.tiny_needle()
    say("select+attention, tiny workload")
    mx, mn = run_meta(qs, wl, sentinel=0.0)
    out, sel, ns = run_fused(qs, wl, mx, mn)
    omx, omn = oracle_meta(oracle, wl, sentinel=0.0)
    osel, ons, osc = oracle.block_select(wl.query, omx, omn, wl.meta_tables, wl.seq_lens, wl.k)
    compare_quest(tnp(sel), tnp(ns), osel, ons, osc, nbs_of(wl), wl.k)
    assert 31 in set(tnp(sel)[0, 0].tolist())                       # the planted needle block
    ref = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, tnp(sel),
                                    tnp(ns), wl.N)
    assert np.abs(out.cpu().numpy() - ref).max() <= 1e-4


# ------------------------------------------------------------------------------------------
# large configurations: full-size launches, every request against the oracle
# ------------------------------------------------------------------------------------------

ORACLE_THREADS = min(8, os.cpu_count() or 1)


def gather_requests(wl, reqs, with_v=True):
    """The given requests as a compact CPU workload (their K, and V, blocks gathered; block
    and metadata tables renumbered; sequence-relative indices unchanged)."""
    BS = wl.BS
    bt = wl.block_tables.cpu()
    mt = wl.meta_tables.cpu()
    sl = wl.seq_lens.cpu()
    msl = wl.meta_seq_lens.cpu()
    nbs = [cdiv(int(sl[b]), BS) for b in reqs]
    phys = torch.cat([bt[b, :nb].long() for b, nb in zip(reqs, nbs)])
    kc = wl.k_cache[phys.to(wl.k_cache.device)].cpu()
    vc = wl.v_cache[phys.to(wl.v_cache.device)].cpu() if with_v and wl.v_cache is not None else None
    nt = torch.zeros((len(reqs), bt.shape[1]), dtype=torch.int32)
    off = 0
    for j, nb in enumerate(nbs):
        nt[j, :nb] = torch.arange(off, off + nb, dtype=torch.int32)
        off += nb
    mnb = [cdiv(nb, BS) for nb in nbs]
    nmt = torch.zeros((len(reqs), mt.shape[1]), dtype=torch.int32)
    off = 0
    for j, m in enumerate(mnb):
        nmt[j, :m] = torch.arange(off, off + m, dtype=torch.int32)
        off += m
    q = wl.query.cpu()[reqs]
    sub = W.Workload(wl.name + "_part", len(reqs), wl.H, wl.N, wl.D, BS, wl.k, q, kc, vc, nt, sl[reqs].clone(),
                     nmt, max(1, off), msl[reqs].clone(),
                     tsmu=None if wl.tsmu is None else wl.tsmu.cpu()[reqs].clone(), flags=wl.flags,
                     sel_heads=wl.sel_heads)
    return sub, nbs


def gather_selected(wl, reqs, sels):
    """CPU copies (K, V, block table) of the given requests holding only the blocks that
    some row of the selections in ``sels`` ([B, rows, k] arrays with their counts) names;
    other table entries point at block 0 and are never read."""
    BS = wl.BS
    bt = wl.block_tables.cpu()
    nbs = [cdiv(int(wl.seq_lens[b]), BS) for b in reqs]
    phys, nt = [], torch.zeros((len(reqs), bt.shape[1]), dtype=torch.int32)
    for j, b in enumerate(reqs):
        used = set()
        for sel, ns in sels:
            for r in range(sel.shape[1]):
                used.update(int(x) for x in sel[b, r, :ns[b, r]] if 0 <= x < nbs[j])
        for blk in sorted(used):
            nt[j, blk] = len(phys)
            phys.append(int(bt[b, blk]))
    idx = torch.tensor(phys if phys else [0], dtype=torch.long, device=wl.k_cache.device)
    return wl.k_cache[idx].cpu(), wl.v_cache[idx].cpu(), nt


def full_size_parity(qs, oracle, wl, settings, chunk):
    """Every request of a full-size workload against the oracle, for each setting (name,
    query [B,H,D], tokens_since_update [B]) on the same KV pools and metadata:

    * metadata rows bit for bit (oracle build over each request's blocks);
    * block scores within 1e-3 relative, selections equal up to near ties (qs_block_select),
      and the fused call's selection bitwise the selection call's;
    * attention at full size on the oracle's selection, and both paths' outputs (the two
      calls and qs_select_attn_decode) on the GPU's selection, against the oracle's
      attention: the contract's 2e-2 and the per-element rounding bound.

    The oracle runs chunk by chunk of requests in a few threads (the C oracle releases the
    interpreter lock). Returns the GPU selections per setting."""
    from concurrent.futures import ThreadPoolExecutor

    B, N, k = wl.B, wl.N, wl.k
    mx = torch.zeros((wl.num_meta_blocks, wl.BS, N, wl.D), dtype=wl.k_cache.dtype, device=DEV)
    mn = torch.zeros_like(mx)
    qs.qs_build_metadata(wl.k_cache, wl.block_tables, wl.meta_seq_lens, wl.meta_tables, mx, mn)
    gpu = {}
    for name, q, ts in settings:
        say(f"{wl.name} [{name}]: select + attention, both paths, full size")
        sc = torch.zeros((B, N, wl.mmbpr * wl.BS), device=DEV)
        sel, ns = qs.qs_block_select(q, mx, mn, wl.meta_tables, wl.seq_lens, k, tokens_since_update=ts,
                                     flags=wl.flags, block_scores=sc)
        out = qs.qs_sparse_attn_decode(q, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, sel, ns)
        fsel = torch.full((B, N, k), -7, dtype=torch.int32, device=DEV)
        fns = torch.full((B, N), -7, dtype=torch.int32, device=DEV)
        fout = qs.qs_select_attn_decode(q, mx, mn, wl.meta_tables, wl.k_cache, wl.v_cache, wl.block_tables,
                                        wl.seq_lens, k, tokens_since_update=ts, flags=wl.flags, selected=fsel,
                                        n_selected=fns)
        torch.cuda.synchronize()
        assert torch.equal(fsel, sel) and torch.equal(fns, ns), f"{name}: fused selection differs"
        gpu[name] = dict(q=q.cpu(), ts=None if ts is None else ts.cpu(), sel=tnp(sel), ns=tnp(ns), sc=tnp(sc),
                         out=out.float().cpu().numpy().astype(np.float64),
                         fout=fout.float().cpu().numpy().astype(np.float64))
    gmx, gmn = bits(tnp(mx)), bits(tnp(mn))
    mt = wl.meta_tables.cpu()
    chunks = [list(range(s, min(B, s + chunk))) for s in range(0, B, chunk)]
    ores = {name: dict(sel=np.zeros((B, N, k), np.int32), ns=np.zeros((B, N), np.int32),
                       sc=np.zeros((B, N, wl.mmbpr * wl.BS))) for name, _, _ in settings}

    def meta_select(reqs, sub, nbs):
        omx, omn = oracle.build_metadata(sub.k_cache, sub.block_tables, sub.meta_seq_lens, sub.meta_tables,
                                         sub.num_meta_blocks)
        bx, bn = bits(omx), bits(omn)
        for j, b in enumerate(reqs):
            for m in range(cdiv(nbs[j], wl.BS)):
                gm, om = int(mt[b, m]), int(sub.meta_tables[j, m])
                assert np.array_equal(gmx[gm], bx[om]) and np.array_equal(gmn[gm], bn[om]), \
                    f"metadata of request {b}, metadata block {m}"
        for name, g in gpu.items():
            ts = None if g["ts"] is None else g["ts"][reqs]
            osel, ons, osc = oracle.block_select(g["q"][reqs], omx, omn, sub.meta_tables, sub.seq_lens, k, tsmu=ts,
                                                 flags=wl.flags)
            r = ores[name]
            r["sel"][reqs], r["ns"][reqs], r["sc"][reqs] = osel, ons, osc

    say(f"{wl.name}: oracle metadata and selections, {len(chunks)} chunks of {chunk} requests")
    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        futs = []
        for reqs in chunks:
            sub, nbs = gather_requests(wl, reqs, with_v=False)
            futs.append(ex.submit(meta_select, reqs, sub, nbs))
            while sum(not f.done() for f in futs) >= ORACLE_THREADS:
                futs[[f.done() for f in futs].index(False)].result()
        for f in futs:
            f.result()
    nbs_all = nbs_of(wl)
    for name, g in gpu.items():
        r = ores[name]
        mask = np.zeros_like(r["sc"], dtype=bool)
        for b, nb in enumerate(nbs_all):
            mask[b, :, :nb] = ~np.isnan(r["sc"][b, :, :nb])
        check_scores(g["sc"], r["sc"], mask)
        near = compare_quest(g["sel"], g["ns"], r["sel"], r["ns"], r["sc"], nbs_all, k)
        say(f"{wl.name} [{name}]: scores and selections of all {B} requests match ({near} near-tie rows)")
        osel_t = torch.from_numpy(r["sel"]).to(DEV)
        ons_t = torch.from_numpy(r["ns"]).to(DEV)
        q = g["q"].to(DEV)
        g["out_o"] = qs.qs_sparse_attn_decode(q, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, osel_t,
                                              ons_t).float().cpu().numpy().astype(np.float64)

    def attend(reqs, kc, vc, nt):
        sl = wl.seq_lens.cpu()[reqs]
        ratios = {}
        for name, g in gpu.items():
            r = ores[name]
            q = g["q"][reqs]
            args = (q, kc, vc, nt, sl)
            pairs = [("oracle selection", r["sel"][reqs], r["ns"][reqs], [("full-size attention", g["out_o"])]),
                     ("GPU selection", g["sel"][reqs], g["ns"][reqs],
                      [("two calls", g["out"]), ("fused call", g["fout"])])]
            for what, sel, ns, outs in pairs:
                ref = oracle.sparse_attn_decode(*args, sel, ns, N)
                tol = attn16_bound(*args, sel, ns, N, ref, q.dtype)
                for label, full in outs:
                    got = full[reqs]
                    err = np.abs(got - ref)
                    assert float(err.max()) <= attn_tol(q.dtype), \
                        f"[{name}] {label} on the {what}, requests {reqs[0]}..{reqs[-1]}: max err {err.max():.3e}"
                    bad = np.argwhere(err > tol)
                    assert bad.size == 0, (f"[{name}] {label} on the {what}: {len(bad)} elements beyond the rounding "
                                           f"bound, first {tuple(bad[0])} err {err[tuple(bad[0])]:.3e} "
                                           f"> {tol[tuple(bad[0])]:.3e}")
                    key = (name, label)
                    ratios[key] = max(ratios.get(key, 0.0), float(np.max(err / tol)), 0.0)
                    ratios[key + ("err",)] = max(ratios.get(key + ("err",), 0.0), float(err.max()))
        return ratios

    say(f"{wl.name}: oracle attention over both selections")
    total = {}
    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        futs = []
        for reqs in chunks:
            sels = []
            for name, g in gpu.items():
                sels += [(g["sel"], g["ns"]), (ores[name]["sel"], ores[name]["ns"])]
            kc, vc, nt = gather_selected(wl, reqs, sels)
            futs.append(ex.submit(attend, reqs, kc, vc, nt))
        for f in futs:
            for key, v in f.result().items():
                total[key] = max(total.get(key, 0.0), v)
    for name, _, _ in settings:
        for label in ("full-size attention", "two calls", "fused call"):
            say(f"{wl.name} [{name}] {label}: all {B} requests, max abs err {total[(name, label, 'err')]:.3e}, "
                f"max err/bound {total[(name, label)]:.3f}")
    return gpu


def test_long_context_full_size_every_request(qs, oracle):
    """Long-context workload (8 requests of 8k..128k tokens, k = 64, sink + window): its own
    queries, whose planted needles dominate each row's softmax, and an independent N(0,1)
    query set on the same pools, where no token dominates and a dropped block would show."""
    wl = W.long_context(device=DEV)
    q2 = W.extra_queries(wl, seed=12)
    gpu = full_size_parity(qs, oracle, wl, [("own queries", wl.query, wl.tsmu), ("independent queries", q2, wl.tsmu)],
                           chunk=1)
    sel, ns = gpu["own queries"]["sel"], gpu["own queries"]["ns"]
    hits = sum(int((t // wl.BS) in set(sel[b, n, :ns[b, n]].tolist())) for b, t in wl.needles for n in range(wl.N))
    say(f"long-context needle recall {hits}/{wl.B * wl.N}")   # reported, not gated


def test_serving_full_size_every_request(qs, oracle):
    """Serving workload (128 requests of 32k tokens, k = 16, sink + window), every request:
    query set 0 with tokens_since_update 0, and query set 1 with a per-request
    tokens_since_update drawn from [0, 127]."""
    wl = W.serving(device=DEV)
    qsets = wl.extra["query_sets"]
    g = torch.Generator().manual_seed(77)
    ts1 = torch.randint(0, 128, (wl.B,), generator=g, dtype=torch.int32).to(DEV)
    full_size_parity(qs, oracle, wl, [("query set 0, tsmu 0", qsets[0].contiguous(), wl.tsmu),
                                      ("query set 1, tsmu drawn", qsets[1].contiguous(), ts1)], chunk=16)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_nontemporal_paths_bitwise_equal_plain_loads(qs, dtype):
    """Calls that stream more than 512 MB read with non-temporal loads, smaller ones with
    plain loads; only the cache policy differs, so the results must be bitwise equal. 256
    requests of 8 blocks (8 KV heads of 8 query heads, k = 4, sink + window forcing): the
    metadata build (an 8.6 GB grid bound), the fused selection + attention (671 MB) and
    the attention alone (537 MB) over all requests, against the same requests in batches
    small enough for plain loads (8 requests per build, 128 per step). Every call has at
    least 1024 rows, so both launch one workgroup per row and merge nothing."""
    B, H, N, BS, L, k = 256, 64, 8, 128, 1024, 4
    ts_list = [int(x) for x in torch.randint(0, 2 * BS, (B,), generator=torch.Generator().manual_seed(9))]
    wl = W.random_case(61, B, H, N, BS, [L] * B, k=k, dtype=dtype, tsmu=ts_list,
                       flags=W.FORCE_SINK | W.FORCE_WINDOW, spare_blocks=0, meta_spare=0).to(DEV)
    say(f"non-temporal vs plain loads, {B} requests, {dtype}")
    shape = (wl.num_meta_blocks, BS, N, wl.D)
    mx, mn = torch.zeros(shape, dtype=dtype, device=DEV), torch.zeros(shape, dtype=dtype, device=DEV)
    qs.qs_build_metadata(wl.k_cache, wl.block_tables, wl.meta_seq_lens, wl.meta_tables, mx, mn)
    mx2, mn2 = torch.zeros_like(mx), torch.zeros_like(mn)
    for b0 in range(0, B, 8):
        r = slice(b0, b0 + 8)
        qs.qs_build_metadata(wl.k_cache, wl.block_tables[r], wl.meta_seq_lens[r], wl.meta_tables[r], mx2, mn2)
    torch.cuda.synchronize()
    assert torch.equal(mx.view(torch.int16), mx2.view(torch.int16))
    assert torch.equal(mn.view(torch.int16), mn2.view(torch.int16))
    sel = torch.empty((B, N, k), dtype=torch.int32, device=DEV)
    ns = torch.empty((B, N), dtype=torch.int32, device=DEV)
    out = qs.qs_select_attn_decode(wl.query, mx, mn, wl.meta_tables, wl.k_cache, wl.v_cache, wl.block_tables,
                                   wl.seq_lens, k, tokens_since_update=wl.tsmu, flags=wl.flags, selected=sel,
                                   n_selected=ns)
    att = qs.qs_sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, sel, ns)
    out2, att2 = torch.empty_like(out), torch.empty_like(out)
    sel2, ns2 = torch.empty_like(sel), torch.empty_like(ns)
    for b0 in range(0, B, 128):
        r = slice(b0, b0 + 128)
        qs.qs_select_attn_decode(wl.query[r], mx, mn, wl.meta_tables[r], wl.k_cache, wl.v_cache,
                                 wl.block_tables[r], wl.seq_lens[r], k, tokens_since_update=wl.tsmu[r],
                                 flags=wl.flags, out=out2[r], selected=sel2[r], n_selected=ns2[r])
        qs.qs_sparse_attn_decode(wl.query[r], wl.k_cache, wl.v_cache, wl.block_tables[r], wl.seq_lens[r],
                                 sel2[r], ns2[r], out=att2[r])
    torch.cuda.synchronize()
    assert int(ns.min()) == k and torch.equal(sel, sel2) and torch.equal(ns, ns2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(att.view(torch.int16), att2.view(torch.int16))
    assert torch.equal(out.view(torch.int16), att.view(torch.int16))


@pytest.mark.parametrize("which", ["long_context", "serving"])
def test_full_size_steps_bitwise_repeatable(qs, which):
    """Determinism at full size: the decode step of the long-context workload (split rows
    merged by the combine pass) and of the serving workload, each run twice through the
    fused call and twice through the two calls, gives bitwise the same selection and
    output each time (and the two paths the same selection)."""
    wl = W.long_context(device=DEV) if which == "long_context" else W.serving(device=DEV)
    say(f"bitwise repeat, {wl.name}")
    mx = torch.zeros((wl.num_meta_blocks, wl.BS, wl.N, wl.D), dtype=wl.k_cache.dtype, device=DEV)
    mn = torch.zeros_like(mx)
    qs.qs_build_metadata(wl.k_cache, wl.block_tables, wl.meta_seq_lens, wl.meta_tables, mx, mn)
    q, ts = wl.query, wl.tsmu
    runs = []
    for _ in range(2):
        sel = torch.empty((wl.B, wl.N, wl.k), dtype=torch.int32, device=DEV)
        ns = torch.empty((wl.B, wl.N), dtype=torch.int32, device=DEV)
        out = qs.qs_select_attn_decode(q, mx, mn, wl.meta_tables, wl.k_cache, wl.v_cache, wl.block_tables,
                                       wl.seq_lens, wl.k, tokens_since_update=ts, flags=wl.flags, selected=sel,
                                       n_selected=ns)
        sel2, ns2 = qs.qs_block_select(q, mx, mn, wl.meta_tables, wl.seq_lens, wl.k, tokens_since_update=ts,
                                       flags=wl.flags)
        out2 = qs.qs_sparse_attn_decode(q, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, sel2, ns2)
        torch.cuda.synchronize()
        runs.append((sel, ns, out.view(torch.int16), sel2, ns2, out2.view(torch.int16)))
    for a, b in zip(runs[0], runs[1]):
        assert torch.equal(a, b)
    assert torch.equal(runs[0][0], runs[0][3]) and torch.equal(runs[0][1], runs[0][4])


def test_workspace_shared_across_shapes_and_operations(qs, oracle):
    """One workspace (filled with garbage first) serves select and attention calls of
    different sizes in turn (no debug score output, so the select scores live in the
    workspace too)."""
    say("shared workspace across shapes")
    ws = torch.full((64 << 20,), 0xA5, dtype=torch.uint8, device=DEV)
    cases = [(51, 4, 64, 8, 128, [128 * 300, 128 * 40, 128 * 999, 128 * 5], 16),
             (52, 1, 16, 8, 32, [32 * 128], 32),
             (53, 2, 32, 8, 64, [64 * 200 + 1, 64 * 90], 8),
             (51, 4, 64, 8, 128, [128 * 300, 128 * 40, 128 * 999, 128 * 5], 16)]
    for seed, B, H, N, BS, lens, k in cases:
        say(f"  shared workspace case seed={seed} B={B} H={H} BS={BS} k={k}")
        wl = W.random_case(seed, B, H, N, BS, lens, k=k, dtype=torch.bfloat16)
        mx, mn = run_meta(qs, wl, sentinel=0.0)
        sel, ns = qs.qs_block_select(wl.query.to(DEV), mx, mn, wl.meta_tables.to(DEV), wl.seq_lens.to(DEV), k,
                                     workspace_buf=ws)
        omx, omn = oracle_meta(oracle, wl, sentinel=0.0)
        osel, ons, osc = oracle.block_select(wl.query, omx, omn, wl.meta_tables, wl.seq_lens, k)
        compare_quest(tnp(sel), tnp(ns), osel, ons, osc, nbs_of(wl), k)
        for sh in (N, H):
            rsel, rns = random_selection(seed, B, sh, k, nbs_of(wl))
            out = qs.qs_sparse_attn_decode(wl.query.to(DEV), wl.k_cache.to(DEV), wl.v_cache.to(DEV),
                                           wl.block_tables.to(DEV), wl.seq_lens.to(DEV), rsel.to(DEV), rns.to(DEV),
                                           sel_heads=sh, workspace_buf=ws)
            ref = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, rsel,
                                            rns, sh)
            assert np.abs(out.float().cpu().numpy() - ref).max() <= 2e-2


def test_graph_replay_matches_eager(qs):
    """The select + attention step captured in a HIP graph and replayed several times,
    with eager work in between, gives bitwise the eager results every time (the path
    records no memset nodes; the kernels are deterministic)."""
    say("graph replay")
    wl = W.random_case(61, 8, 64, 8, 128, [128 * 100 + 5] * 4 + [128 * 40] * 4, k=16, dtype=torch.bfloat16,
                       flags=W.FORCE_SINK | W.FORCE_WINDOW, tsmu=[3] * 8)
    wl = wl.to(DEV)
    mx = torch.zeros((wl.num_meta_blocks, wl.BS, wl.N, wl.D), dtype=torch.bfloat16, device=DEV)
    mn = torch.zeros_like(mx)
    qs.qs_build_metadata(wl.k_cache, wl.block_tables, wl.meta_seq_lens, wl.meta_tables, mx, mn)
    sel = torch.empty((wl.B, wl.N, wl.k), dtype=torch.int32, device=DEV)
    ns = torch.empty((wl.B, wl.N), dtype=torch.int32, device=DEV)
    out = torch.empty((wl.B, wl.H, wl.D), dtype=torch.bfloat16, device=DEV)
    ws1 = torch.empty(qs.block_select_workspace_bytes(wl.B, wl.N, wl.BS, wl.mmbpr), dtype=torch.uint8, device=DEV)
    ws2 = torch.empty(qs.sparse_attn_workspace_bytes(wl.B, wl.H, wl.N, wl.D, wl.N, wl.k), dtype=torch.uint8,
                      device=DEV)

    def step():
        qs.qs_block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, wl.k, tokens_since_update=wl.tsmu,
                           flags=wl.flags, selected=sel, n_selected=ns, workspace_buf=ws1)
        qs.qs_sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, sel, ns,
                                 out=out, workspace_buf=ws2)

    step()
    torch.cuda.synchronize()
    want = (sel.clone(), ns.clone(), out.clone())
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            step()
    torch.cuda.current_stream().wait_stream(cs)
    for rep in range(3):
        sel.fill_(-7)
        out.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, want[0]) and torch.equal(ns, want[1]), rep
        assert torch.equal(out.view(torch.int16), want[2].view(torch.int16)), rep
        step()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want[2].view(torch.int16))


def test_two_streams_run_concurrently(qs):
    """Two different workloads issued on two streams at once, each a few times over (Quest
    select + attention in one call, and the probe selection + attention in one call), give
    bitwise what each gives alone: the binding keeps a workspace per (stream, operation),
    so concurrent calls never share scratch memory."""
    say("two streams")
    wa = W.random_case(71, 8, 32, 8, 64, [64 * 90 + 7] * 8, k=12, dtype=torch.bfloat16,
                       flags=W.FORCE_SINK | W.FORCE_WINDOW, tsmu=[9] * 8).to(DEV)
    wb = W.random_case(72, 4, 16, 8, 32, [32 * 120 + 3] * 4, k=16, dtype=torch.float32,
                       with_importance=True).to(DEV)
    mx, mn = run_meta(qs, wa, sentinel=0.0)

    def call_a():
        return qs.qs_select_attn_decode(wa.query, mx, mn, wa.meta_tables, wa.k_cache, wa.v_cache, wa.block_tables,
                                        wa.seq_lens, wa.k, tokens_since_update=wa.tsmu, flags=wa.flags)

    def call_b():
        return qs.qs_probe_attn_decode(wb.query, wb.k_cache, wb.v_cache, wb.block_tables, wb.seq_lens, wb.k,
                                       importance=wb.importance, n_probe=8, flags=qs.QS_RECENCY)

    want_a, want_b = call_a().clone(), call_b().clone()
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    outs_a, outs_b = [], []
    for _ in range(4):
        with torch.cuda.stream(sa):
            outs_a.append(call_a())
        with torch.cuda.stream(sb):
            outs_b.append(call_b())
    torch.cuda.synchronize()
    for o in outs_a:
        assert torch.equal(o.view(torch.int16), want_a.view(torch.int16))
    for o in outs_b:
        assert torch.equal(o.view(torch.int32), want_b.view(torch.int32))


def test_graphs_of_one_operation_replay_concurrently(qs):
    """Two graphs of the same operation captured on torch's default capture stream, with no
    workspace passed (each captured call gets scratch of its own from its graph's pool),
    replayed at the same time on two streams, several times over: each replay gives bitwise
    its own eager result."""
    say("two graphs of one operation replayed concurrently")
    was = []
    for seed in (63, 64):
        wl = W.random_case(seed, 4, 32, 8, 64, [64 * 150 + 3, 64 * 90, 64 * 200 + 17, 64 * 40], k=12,
                           dtype=torch.bfloat16, flags=W.FORCE_SINK | W.FORCE_WINDOW, tsmu=[3, 0, 5, 1]).to(DEV)
        mx, mn = run_meta(qs, wl, sentinel=0.0)
        out = torch.empty((wl.B, wl.H, wl.D), dtype=torch.bfloat16, device=DEV)
        was.append((wl, mx, mn, out))

    def call(i):
        wl, mx, mn, out = was[i]
        qs.qs_select_attn_decode(wl.query, mx, mn, wl.meta_tables, wl.k_cache, wl.v_cache, wl.block_tables,
                                 wl.seq_lens, wl.k, tokens_since_update=wl.tsmu, flags=wl.flags, out=out)

    want = []
    for i in range(2):
        call(i)
        torch.cuda.synchronize()
        want.append(was[i][3].clone())
    graphs = []
    for i in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(i)
        graphs.append(g)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(4):
        for i in range(2):
            was[i][3].fill_(5.0)
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            graphs[0].replay()
        with torch.cuda.stream(sb):
            graphs[1].replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(was[i][3].view(torch.int16), want[i].view(torch.int16)), (rep, i)


def test_workspace_cache_grows_twofold(qs):
    """The binding's cached workspace of one (device, stream, operation) is reused while it
    suffices and grows at least twofold when it does not, so the replaced buffers it keeps
    allocated (a captured graph may hold their addresses) stay under twice the largest."""
    op = "growth_check"
    before = len(qs._retired)
    w1 = qs.workspace(1000, DEV, op)
    assert w1.numel() >= 1000 and qs.workspace(900, DEV, op) is w1
    sizes = [w1.numel()]
    for n in range(1001, 200000, 997):   # slowly growing requests
        w = qs.workspace(n, DEV, op)
        assert w.numel() >= n
        if w.numel() != sizes[-1]:
            sizes.append(w.numel())
    assert all(b >= 2 * a for a, b in zip(sizes, sizes[1:]))
    retired = len(qs._retired) - before
    assert retired == len(sizes) - 1 <= 8
    assert sum(sizes[:-1]) < sizes[-1]


def test_graph_replay_probe_path(qs):
    """Page 1's path captured in a HIP graph: a metadata refresh, the prefill importance, the
    probe selection and fp32 attention with one selection row per query head, and the fused
    probe selection + attention call beside them. No workspace is passed, so every captured
    call takes a workspace of its own from the graph's memory pool. Three replays, with the
    same eager calls (on the binding's cached workspaces) between them, give bitwise the
    eager results."""
    say("graph replay, probe path")
    wl = W.random_case(62, 2, 16, 8, 32, [32 * 60 + 5, 32 * 33], k=12, dtype=torch.float32, with_v=True)
    pq = W.prefill_queries(wl, 62).to(DEV)
    wl = wl.to(DEV)
    B, H, N, BS = wl.B, wl.H, wl.N, wl.BS
    mx = torch.zeros((wl.num_meta_blocks, BS, N, wl.D), dtype=torch.float32, device=DEV)
    mn = torch.zeros_like(mx)
    last = torch.tensor([cdiv(int(x), BS) - 1 for x in wl.seq_lens.cpu().tolist()], dtype=torch.int32, device=DEV)
    imp = torch.empty((B, pq.shape[1]), dtype=torch.float32, device=DEV)
    psel = torch.empty((B, H, wl.k), dtype=torch.int32, device=DEV)
    pns = torch.empty((B, H), dtype=torch.int32, device=DEV)
    out = torch.empty((B, H, wl.D), dtype=torch.float32, device=DEV)
    fsel, fns, fout = torch.empty_like(psel), torch.empty_like(pns), torch.empty_like(out)

    def step():
        qs.qs_update_metadata(wl.k_cache, wl.block_tables, wl.seq_lens, last, 1, wl.meta_tables, mx, mn)
        qs.qs_prefill_importance(pq, wl.k_cache, wl.block_tables, wl.seq_lens, importance=imp)
        qs.qs_probe_select(wl.query, wl.k_cache, wl.block_tables, wl.seq_lens, wl.k, importance=imp, n_probe=8,
                           flags=qs.QS_RECENCY, selected=psel, n_selected=pns)
        qs.qs_sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, psel, pns,
                                 sel_heads=H, out=out)
        qs.qs_probe_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, wl.k, importance=imp,
                                n_probe=8, flags=qs.QS_RECENCY, out=fout, selected=fsel, n_selected=fns)

    step()
    torch.cuda.synchronize()
    assert torch.equal(fsel, psel) and torch.equal(fns, pns)
    assert float((fout - out).abs().max()) <= 1e-5
    want = [t.clone() for t in (mx, mn, imp, psel, pns, out, fsel, fns, fout)]
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            step()
    torch.cuda.current_stream().wait_stream(cs)
    for rep in range(3):
        for t in (mx, mn, imp, out, fout):
            t.fill_(5.0)
        psel.fill_(-7)
        fsel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (mx, mn, imp, psel, pns, out, fsel, fns, fout)
        names = ("maxblocks", "minblocks", "importance", "selected", "n_selected", "out", "fused selected",
                 "fused n_selected", "fused out")
        for name, a, b in zip(names, got, want):
            if name in ("maxblocks", "minblocks"):  # only the refreshed rows are defined after the fill
                rows = [(int(wl.meta_tables[bb, int(last[bb]) // BS]), int(last[bb]) % BS) for bb in range(B)]
                for m, r in rows:
                    assert torch.equal(a[m, r].view(torch.int32), b[m, r].view(torch.int32)), (rep, name)
            else:
                assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (rep, name)
        step()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want[5].view(torch.int32))


# ------------------------------------------------------------------------------------------
# page-3 call shapes (top_kv_block_amd.quest_ops)
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_page3_wrappers(qs, oracle, dtype):
    """The page's example shapes (B=20, H=32, N=8, BS=128, MMBPR=1, k=8) through the page-3
    names, in fp16 and bf16, against the oracle; the forcing variant with a scalar
    tokens_since_metadata_update of 0 and of -1 (off)."""
    from top_kv_block_amd import quest_ops as Q
    say(f"page-3 wrappers dtype={dtype}")
    B, H, N, BS, k = 20, 32, 8, 128, 8
    wl = W.random_case(81, B, H, N, BS, [BS * BS] * 10 + [BS * 100 + 17] * 10, k=k, dtype=dtype, dist="uniform",
                       with_v=False)
    kc, bt, mt, sl = wl.k_cache.to(DEV), wl.block_tables.to(DEV), wl.meta_tables.to(DEV), wl.seq_lens.to(DEV)
    mx = torch.zeros((wl.num_meta_blocks, BS, N, wl.D), dtype=dtype, device=DEV)
    mn = torch.zeros_like(mx)
    Q.quest_prefill_metadata(kc, sl, bt, mt, mx, mn)
    omx, omn = oracle.build_metadata(wl.k_cache, wl.block_tables, wl.seq_lens, wl.meta_tables, wl.num_meta_blocks)
    assert np.array_equal(bits(tnp(mx)), bits(omx)) and np.array_equal(bits(tnp(mn)), bits(omn))
    q = wl.query.to(DEV)
    ids = Q.quest_block_select_paged(q, mx, mn, mt, sl, k)
    assert ids.shape == (B, N, k) and ids.dtype == torch.int32
    osel, ons, osc = oracle.block_select(wl.query, omx, omn, wl.meta_tables, wl.seq_lens, k)
    compare_quest(tnp(ids), ons, osel, ons, osc, nbs_of(wl), k)
    ids2 = torch.zeros((B, N, k), dtype=torch.int32, device=DEV)
    Q.quest_block_select_paged_in_out(q, mx, mn, mt, sl, ids2)
    assert torch.equal(ids, ids2)
    for tsmu in (0, -1):
        Q.quest_block_select_paged_in_out_w(q, mx, mn, mt, sl, tsmu, ids2)
        osel, ons, osc = oracle.block_select(wl.query, omx, omn, wl.meta_tables, wl.seq_lens, k,
                                             tsmu=torch.full((B,), tsmu, dtype=torch.int32),
                                             flags=W.FORCE_SINK | W.FORCE_WINDOW)
        compare_quest(tnp(ids2), ons, osel, ons, osc, nbs_of(wl), k)
        if tsmu == 0:
            assert all(0 in set(r.tolist()) for r in tnp(ids2).reshape(-1, k))      # sink forced


# ------------------------------------------------------------------------------------------
# fused probe selection + attention (qs_probe_attn_decode)
# ------------------------------------------------------------------------------------------

PROBE_ATTN_CASES = [
    # seed, B, H, N, BS, lens, k, dtype, importance, flags, n_probe
    (401, 2, 16, 8, 32, [32 * 128, 32 * 3 + 1], 32, torch.float32, True, W.RECENCY, 8),  # page-1 shape, ragged
    (402, 3, 8, 2, 16, [500, 0, 33], 5, torch.float32, False, W.RECENCY, 3),             # empty request, no importance
    (403, 2, 6, 3, 64, [1000, 64], 40, torch.bfloat16, True, 0, 8),                      # k > nb
    (404, 4, 4, 4, 128, [3000, 128 * 20 + 1, 7, 2000], 12, torch.float16, True, W.RECENCY, 64),
    (405, 64, 32, 8, 16, [16 * 40 + 3] * 64, 4, torch.float32, True, W.RECENCY, 8),     # 2048 rows: no slot splits
    (406, 1, 2, 1, 16, [16 * 4096], 100, torch.float32, True, W.RECENCY, 8),            # a 4096-block row
    (407, 1, 2, 1, 16, [16 * 4096], 4096, torch.float32, True, W.RECENCY, 8),           # k at its maximum: all blocks
    (408, 2, 4, 2, 16, [16 * 50, 16 * 50 - 9], 4096, torch.float32, False, W.RECENCY, 2),  # k far above nb
]


@pytest.mark.parametrize("case", PROBE_ATTN_CASES, ids=lambda c: f"seed{c[0]}")
def test_probe_attn_matches_probe_select_and_oracle(qs, oracle, case):
    """The fused call's selection is bitwise qs_probe_select's; its output matches the
    oracle's attention over that selection (one row per query head)."""
    seed, B, H, N, BS, lens, k, dtype, use_imp, flags, n_probe = case
    say(f"probe+attn seed={seed} B={B} H={H} N={N} BS={BS} k={k} dtype={dtype} imp={use_imp} flags={flags}")
    wl = W.random_case(seed, B, H, N, BS, lens, k=k, dtype=dtype, with_importance=use_imp)
    imp = wl.importance.to(DEV) if use_imp else None
    q, kc, vc, bt, sl = (t.to(DEV) for t in (wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens))
    sel, ns = qs.qs_probe_select(q, kc, bt, sl, k, importance=imp, n_probe=n_probe, flags=flags)
    fsel = torch.full((B, H, k), -7, dtype=torch.int32, device=DEV)
    fns = torch.full((B, H), -7, dtype=torch.int32, device=DEV)
    out = qs.qs_probe_attn_decode(q, kc, vc, bt, sl, k, importance=imp, n_probe=n_probe, flags=flags,
                                  selected=fsel, n_selected=fns)
    torch.cuda.synchronize()
    assert torch.equal(fsel, sel) and torch.equal(fns, ns), "fused selection differs from qs_probe_select"
    o = oracle.probe_select(wl.query, wl.k_cache, wl.block_tables, wl.seq_lens, k, N,
                            importance=wl.importance if use_imp else None, n_probe=n_probe, flags=flags)
    compare_probe(tnp(fsel), tnp(fns), o, nbs_of(wl), k)
    ref = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, tnp(fsel),
                                    tnp(fns), H)
    check_attn(out, ref, wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, tnp(fsel), tnp(fns), H,
               f"probe+attn seed={seed}")
    # without the selection outputs: the same attention, bitwise
    out2 = qs.qs_probe_attn_decode(q, kc, vc, bt, sl, k, importance=imp, n_probe=n_probe, flags=flags)
    assert torch.equal(out2.view(torch.int16 if dtype != torch.float32 else torch.int32),
                       out.view(torch.int16 if dtype != torch.float32 else torch.int32))


PROBE_ATTN_I8_CASES = [
    # seed, B, H, N, BS, lens, k, query dtype, probe K dtype, importance, flags, n_probe
    (411, 2, 16, 8, 32, [32 * 128, 32 * 3 + 1], 32, torch.float32, torch.float32, True, W.RECENCY, 8),  # page-1 shape
    (412, 3, 8, 2, 16, [500, 0, 33], 5, torch.float32, torch.float32, False, W.RECENCY, 3),          # empty request
    (413, 2, 6, 3, 64, [1000, 64], 40, torch.bfloat16, torch.bfloat16, True, 0, 8),                  # k > nb, bf16
    (414, 64, 32, 8, 16, [16 * 40 + 3] * 64, 4, torch.float32, torch.float32, True, W.RECENCY, 8),  # no slot splits
    (415, 2, 16, 8, 32, [32 * 200 + 5, 32 * 7], 9, torch.float16, torch.float32, True, W.RECENCY, 8),  # mixed types
]


@pytest.mark.parametrize("case", PROBE_ATTN_I8_CASES, ids=lambda c: f"seed{c[0]}")
def test_probe_attn_int8_matches_two_calls_and_oracle(qs, oracle, case):
    """The fused probe call over an int8 KV cache: the probes read the float K, the attention
    the int8 copy with its scales. The selection is bitwise qs_probe_select's on the float K;
    the output matches qs_sparse_attn_decode over the int8 cache on that selection and the
    oracle's int8 attention (fp32 query: within 2e-5, i.e. the int32 dots and the query
    quantiser bit for bit in effect; 16-bit query: the output dtype's tolerance)."""
    seed, B, H, N, BS, lens, k, qd, pkd, use_imp, flags, n_probe = case
    say(f"probe+attn int8 seed={seed} B={B} H={H} N={N} BS={BS} k={k} q={qd} probe K={pkd}")
    wl = W.random_case(seed, B, H, N, BS, lens, k=k, dtype=torch.float32, with_importance=use_imp, int8=True)
    q = wl.query.to(qd)
    pk = wl.k_cache.to(pkd)
    imp = wl.importance.to(DEV) if use_imp else None
    d = lambda t: t.to(DEV)
    sel, ns = qs.qs_probe_select(d(q), d(pk), d(wl.block_tables), d(wl.seq_lens), k, importance=imp,
                                 n_probe=n_probe, flags=flags)
    two = qs.qs_sparse_attn_decode(d(q), d(wl.k_i8), d(wl.v_i8), d(wl.block_tables), d(wl.seq_lens), sel, ns,
                                   sel_heads=H, k_scale=d(wl.k_scale), v_scale=d(wl.v_scale))
    fsel = torch.full((B, H, k), -7, dtype=torch.int32, device=DEV)
    fns = torch.full((B, H), -7, dtype=torch.int32, device=DEV)
    out = qs.qs_probe_attn_decode(d(q), d(wl.k_i8), d(wl.v_i8), d(wl.block_tables), d(wl.seq_lens), k,
                                  importance=imp, n_probe=n_probe, flags=flags, selected=fsel, n_selected=fns,
                                  k_scale=d(wl.k_scale), v_scale=d(wl.v_scale), probe_k=d(pk))
    torch.cuda.synchronize()
    assert torch.equal(fsel, sel) and torch.equal(fns, ns), "fused selection differs from qs_probe_select"
    o = oracle.probe_select(q, pk, wl.block_tables, wl.seq_lens, k, N,
                            importance=wl.importance if use_imp else None, n_probe=n_probe, flags=flags)
    compare_probe(tnp(fsel), tnp(fns), o, nbs_of(wl), k)
    ref = oracle.sparse_attn_decode(q, wl.k_i8, wl.v_i8, wl.block_tables, wl.seq_lens, tnp(fsel), tnp(fns), H,
                                    k_scale=wl.k_scale, v_scale=wl.v_scale)
    tol = 2e-5 if qd == torch.float32 else attn_tol(qd)
    for what, got in (("fused", out), ("two calls", two)):
        err = float(np.abs(got.float().cpu().numpy() - ref).max()) if ref.size else 0.0
        assert err <= tol, f"{what}: int8 attention err {err:.3e} > {tol}"


def test_probe_decode_loop(qs, oracle):
    """Page 1's decode path over growing lengths: per step one more token per request and the
    fused probe selection + attention (prefill importance over the prompt only, so the new
    tokens add nothing to it; recency forces the newest block), every step's selection and
    output against the oracle."""
    BS, N, H, k = 16, 4, 8, 7
    prompt = [16 * 18 + 3, 16 * 10 + 15]
    steps = BS + 9
    final = [x + steps for x in prompt]
    B = len(prompt)
    say(f"probe decode loop BS={BS} prompt={prompt} steps={steps}")
    wl = W.random_case(32, B, H, N, BS, final, k=k, dtype=torch.float32, with_importance=True)
    imp = wl.importance[:, :max(prompt)].contiguous()     # the prefill's importance row
    for b, L in enumerate(prompt):
        imp[b, L:] = 0.0
    kc, vc, bt = wl.k_cache.to(DEV), wl.v_cache.to(DEV), wl.block_tables.to(DEV)
    gen = torch.Generator().manual_seed(32)
    cur = list(prompt)
    for step in range(steps):
        cur = [x + 1 for x in cur]
        q = torch.randn((B, H, wl.D), generator=gen)
        sl = torch.tensor(cur, dtype=torch.int32)
        sel = torch.full((B, H, k), -7, dtype=torch.int32, device=DEV)
        ns = torch.full((B, H), -7, dtype=torch.int32, device=DEV)
        out = qs.qs_probe_attn_decode(q.to(DEV), kc, vc, bt, sl.to(DEV), k, importance=imp.to(DEV), n_probe=8,
                                      flags=W.RECENCY, selected=sel, n_selected=ns)
        torch.cuda.synchronize()
        o = oracle.probe_select(q, wl.k_cache, wl.block_tables, sl, k, N, importance=imp, n_probe=8, flags=W.RECENCY)
        nbs = [cdiv(c, BS) for c in cur]
        compare_probe(tnp(sel), tnp(ns), o, nbs, k)
        assert all(int(nb - 1) in set(tnp(sel)[b, h, :tnp(ns)[b, h]].tolist())
                   for b, nb in enumerate(nbs) for h in range(H)), "recency: the newest block is picked"
        ref = oracle.sparse_attn_decode(q, wl.k_cache, wl.v_cache, wl.block_tables, sl, tnp(sel), tnp(ns), H)
        err = float(np.abs(out.cpu().numpy() - ref).max())
        assert err <= 1e-4, f"step {step}: attention err {err:.3e}"


def test_probe_attn_page1_k_sweep(qs, oracle):
    """Page 1's probe workload (fp32, 16 heads, 128 blocks of 32, importance, recency) for
    k = 1 .. 32: fused selection bitwise the two calls', output within 1e-4 of the oracle;
    and the same over the workload's int8 copy (probes on the fp32 K), within 2e-5 of the
    oracle's int8 attention."""
    wl = W.page1_probe()
    q, kc, vc, bt, sl, imp = (t.to(DEV) for t in (wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens,
                                                   wl.importance))
    k8, v8, ks, vs = (t.to(DEV) for t in (wl.k_i8, wl.v_i8, wl.k_scale, wl.v_scale))
    for k in (1, 2, 4, 8, 16, 32):
        say(f"probe+attn int8, page-1 workload, k={k}")
        sel, ns = qs.qs_probe_select(q, kc, bt, sl, k, importance=imp, n_probe=8, flags=W.RECENCY)
        fsel, fns = torch.empty_like(sel), torch.empty_like(ns)
        out = qs.qs_probe_attn_decode(q, k8, v8, bt, sl, k, importance=imp, n_probe=8, flags=W.RECENCY,
                                      selected=fsel, n_selected=fns, k_scale=ks, v_scale=vs, probe_k=kc)
        torch.cuda.synchronize()
        assert torch.equal(fsel, sel) and torch.equal(fns, ns)
        ref = oracle.sparse_attn_decode(wl.query, wl.k_i8, wl.v_i8, wl.block_tables, wl.seq_lens, tnp(sel), tnp(ns),
                                        wl.H, k_scale=wl.k_scale, v_scale=wl.v_scale)
        err = float(np.abs(out.cpu().numpy() - ref).max())
        assert err <= 2e-5, f"int8 k={k}: err {err:.3e}"
    for k in (1, 2, 4, 8, 16, 32):
        say(f"probe+attn, page-1 workload, k={k}")
        sel, ns = qs.qs_probe_select(q, kc, bt, sl, k, importance=imp, n_probe=8, flags=W.RECENCY)
        fsel = torch.empty_like(sel)
        fns = torch.empty_like(ns)
        out = qs.qs_probe_attn_decode(q, kc, vc, bt, sl, k, importance=imp, n_probe=8, flags=W.RECENCY,
                                      selected=fsel, n_selected=fns)
        torch.cuda.synchronize()
        assert torch.equal(fsel, sel) and torch.equal(fns, ns)
        ref = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, tnp(sel),
                                        tnp(ns), wl.H)
        err = float(np.abs(out.cpu().numpy() - ref).max())
        assert err <= 1e-4, f"k={k}: err {err:.3e}"


# ------------------------------------------------------------------------------------------
# prefill importance (qs_prefill_importance)
# ------------------------------------------------------------------------------------------

def check_importance(got, want, what):
    """fp32 matrix-core evaluation against the fp64 oracle: relative 2e-4 plus 1e-6."""
    err = np.abs(got.astype(np.float64) - want)
    bad = err > 2e-4 * np.abs(want) + 1e-6
    assert not bad.any(), f"{what}: {bad.sum()} entries off, worst {err.max():.3e}"


IMP_CASES = [
    # seed, B, H, N, BS, lens, dtype, max_len, stride, scale
    (101, 2, 4, 2, 16, [37, 50], torch.float32, 50, 64, 0.0),
    (102, 3, 8, 4, 32, [200, 1, 0], torch.bfloat16, 203, 203, 0.0),
    (103, 1, 16, 8, 32, [640], torch.float16, 640, 700, 0.2),
    (104, 2, 6, 3, 64, [129, 300], torch.float32, 301, 250, 0.0),   # stride shorter than a prompt
    (105, 1, 2, 1, 128, [1000], torch.bfloat16, 1000, 1000, 0.0),
    (106, 2, 3, 1, 16, [1500, 700], torch.bfloat16, 1500, 1500, 0.0),  # 8 chunks of 192 keys, ragged
]


@pytest.mark.parametrize("case", IMP_CASES, ids=lambda c: f"seed{c[0]}")
def test_prefill_importance_random(qs, oracle, case):
    seed, B, H, N, BS, lens, dtype, max_len, stride, scale = case
    say(f"prefill importance seed={seed} B={B} H={H} N={N} BS={BS} lens={lens} dtype={dtype}")
    wl = W.random_case(seed, B, H, N, BS, lens, k=2, dtype=dtype, with_v=False)
    q = W.prefill_queries(wl, seed, max_len=max_len)
    imp, himp = qs.qs_prefill_importance(q.to(DEV), wl.k_cache.to(DEV), wl.block_tables.to(DEV), wl.seq_lens.to(DEV),
                                         softmax_scale=scale, importance_stride=stride, with_heads=True)
    torch.cuda.synchronize()
    oimp, ohimp = oracle.prefill_importance(q, wl.k_cache, wl.block_tables, wl.seq_lens, N, softmax_scale=scale,
                                            stride=stride)
    check_importance(tnp(imp), oimp, "importance")
    check_importance(tnp(himp), ohimp, "head importance")
    for b, L in enumerate(lens):
        assert not tnp(imp)[b, L:].any() and not tnp(himp)[b, :, L:].any()
    # deterministic: a second run is bitwise identical
    imp2 = qs.qs_prefill_importance(q.to(DEV), wl.k_cache.to(DEV), wl.block_tables.to(DEV), wl.seq_lens.to(DEV),
                                    softmax_scale=scale, importance_stride=stride)
    assert torch.equal(imp, imp2)


@pytest.mark.parametrize("case", [(111, 2, 4, 2, 16, [1000, 517], 1000), (112, 1, 3, 3, 64, [63], 64),
                                  (113, 3, 2, 1, 32, [0, 300, 1], 301)], ids=lambda c: f"seed{c[0]}")
def test_prefill_importance_fp32_stored_and_recomputed_scores(qs, oracle, case):
    """fp32 inputs with the full workspace (the first pass stores its causal score tiles and
    the second streams them back) and with the minimum one (the second pass recomputes the
    scores): both against the oracle, ragged prompts and an empty one included."""
    seed, B, H, N, BS, lens, max_len = case
    say(f"prefill importance stored/recomputed seed={seed} B={B} H={H} lens={lens}")
    wl = W.random_case(seed, B, H, N, BS, lens, k=2, dtype=torch.float32, with_v=False)
    q = W.prefill_queries(wl, seed, max_len=max_len)
    t16 = (max_len + 15) // 16
    full = qs.prefill_importance_workspace_bytes(B, H, max_len)
    score = B * H * t16 * (t16 + 1) // 2 * 1024
    assert full > score > 0
    args = (q.to(DEV), wl.k_cache.to(DEV), wl.block_tables.to(DEV), wl.seq_lens.to(DEV))
    oimp, ohimp = oracle.prefill_importance(q, wl.k_cache, wl.block_tables, wl.seq_lens, N)
    for nb in (full, full - score):
        ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
        imp, himp = qs.qs_prefill_importance(*args, with_heads=True, workspace_buf=ws)
        torch.cuda.synchronize()
        check_importance(tnp(imp), oimp, f"importance ({nb} workspace bytes)")
        check_importance(tnp(himp), ohimp, f"head importance ({nb} workspace bytes)")


def test_prefill_importance_fp32_skipped_blocks(qs):
    """Table entries out of range (the plain build skips their blocks): the skipped keys get
    importance 0 and every other value stays finite, identically placed on the stored-score
    and recompute paths, which agree (the oracle refuses such input, so the two paths are
    compared with each other)."""
    B, H, N, BS, lens = 2, 4, 2, 16, [200, 131]
    say(f"prefill importance skipped blocks B={B} H={H} lens={lens}")
    wl = W.random_case(114, B, H, N, BS, lens, k=2, dtype=torch.float32, with_v=False)
    q = W.prefill_queries(wl, 114, max_len=200)
    bt = wl.block_tables.clone()
    nkv = wl.k_cache.shape[0]
    bt[0, 3] = -1    # keys 48 .. 63 of request 0
    bt[1, 0] = nkv   # keys 0 .. 15 of request 1 (row 0's only key)
    bt[1, 8] = -5    # keys 128 .. 130 of request 1 (its last, partial block)
    args = (q.to(DEV), wl.k_cache.to(DEV), bt.to(DEV), wl.seq_lens.to(DEV))
    t16 = (200 + 15) // 16
    full = qs.prefill_importance_workspace_bytes(B, H, 200)
    outs = []
    for nb in (full, full - B * H * t16 * (t16 + 1) // 2 * 1024):
        ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
        ws.fill_(0x7f)  # leftover bytes read as a large finite value
        imp, himp = qs.qs_prefill_importance(*args, with_heads=True, workspace_buf=ws)
        torch.cuda.synchronize()
        outs.append((tnp(imp).astype(np.float64), tnp(himp).astype(np.float64)))
    for imp, himp in outs:
        assert np.isfinite(imp).all() and np.isfinite(himp).all()
        assert not imp[0, 48:64].any() and not imp[1, 0:16].any() and not imp[1, 128:131].any()
        assert imp[0, :48].all() and imp[0, 64:200].all() and imp[1, 16:128].all()
    for a, b in zip(outs[0], outs[1]):
        err = np.abs(a - b)
        assert (err <= 2e-4 * np.abs(b) + 1e-6).all(), f"stored vs recomputed: worst {err.max():.3e}"


def test_prefill_importance_page1_prompt_sampled_heads(qs, oracle):
    """The page-1 probe workload's prefill (4096 tokens, 16 heads, fp32): every head on the GPU, heads 0 and 15
    against the oracle, and the row-mass identity (the importance sums to H * L)."""
    wl, q = W.page1_probe_prefill()
    say("prefill importance, page-1 prompt (4096 tokens)")
    imp, himp = qs.qs_prefill_importance(q.to(DEV), wl.k_cache.to(DEV), wl.block_tables.to(DEV), wl.seq_lens.to(DEV),
                                         with_heads=True)
    torch.cuda.synchronize()
    g, gh = tnp(imp), tnp(himp)
    L = int(wl.seq_lens[0])
    assert abs(g[0].astype(np.float64).sum() - wl.H * L) <= 1e-4 * wl.H * L
    for lo in (0, 15):
        _, oh = oracle.prefill_importance(q, wl.k_cache, wl.block_tables, wl.seq_lens, wl.N, heads=(lo, lo + 1))
        check_importance(gh[:, lo], oh[:, lo], f"head {lo}")


def test_prefill_importance_one_chunk_sampled_heads(qs, oracle):
    """A job large enough to balance without chunks (2 requests x 32 heads x 128 tiles of 64
    rows): one chunk per tile. Ragged lengths (8192 and 5000 tokens), bf16; heads 0 and 31
    against the oracle, zeros past each prompt."""
    B, H, N, BS, lens = 2, 32, 8, 64, [8192, 5000]
    say(f"prefill importance one chunk B={B} H={H} lens={lens}")
    wl = W.random_case(107, B, H, N, BS, lens, k=2, dtype=torch.bfloat16, with_v=False)
    q = W.prefill_queries(wl, 107, max_len=max(lens))
    imp, himp = qs.qs_prefill_importance(q.to(DEV), wl.k_cache.to(DEV), wl.block_tables.to(DEV), wl.seq_lens.to(DEV),
                                         with_heads=True)
    torch.cuda.synchronize()
    g, gh = tnp(imp), tnp(himp)
    for b, L in enumerate(lens):
        assert not g[b, L:].any() and not gh[b, :, L:].any()
        assert abs(g[b, :L].astype(np.float64).sum() - H * L) <= 1e-4 * H * L
    for lo in (0, H - 1):
        _, oh = oracle.prefill_importance(q, wl.k_cache, wl.block_tables, wl.seq_lens, N, heads=(lo, lo + 1))
        check_importance(gh[:, lo], oh[:, lo], f"head {lo}")


@pytest.mark.parametrize("lens,k", [([128 * 100 + 5] * 4 + [128 * 40] * 4, 16),        # one kernel, slot splits
                                    ([128 * 700, 128 * 300 + 9], 48)],                  # scoring grid + top-k/attention
                         ids=["one_kernel", "prescored"])
def test_graph_replay_fused_matches_eager(qs, lens, k):
    """qs_select_attn_decode captured in a HIP graph (each mode, with the combine pass) and
    replayed with eager work in between: bitwise the eager results every time."""
    say(f"graph replay fused k={k}")
    B = len(lens)
    wl = W.random_case(62, B, 64, 8, 128, lens, k=k, dtype=torch.bfloat16, flags=W.FORCE_SINK | W.FORCE_WINDOW,
                       tsmu=[5] * B).to(DEV)
    mx = torch.zeros((wl.num_meta_blocks, wl.BS, wl.N, wl.D), dtype=torch.bfloat16, device=DEV)
    mn = torch.zeros_like(mx)
    qs.qs_build_metadata(wl.k_cache, wl.block_tables, wl.meta_seq_lens, wl.meta_tables, mx, mn)
    sel = torch.empty((wl.B, wl.N, wl.k), dtype=torch.int32, device=DEV)
    ns = torch.empty((wl.B, wl.N), dtype=torch.int32, device=DEV)
    out = torch.empty((wl.B, wl.H, wl.D), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(qs.select_attn_workspace_bytes(wl.B, wl.H, wl.N, wl.BS, wl.mmbpr, wl.k, qs.QS_BF16),
                     dtype=torch.uint8, device=DEV)

    def step():
        qs.qs_select_attn_decode(wl.query, mx, mn, wl.meta_tables, wl.k_cache, wl.v_cache, wl.block_tables,
                                 wl.seq_lens, wl.k, tokens_since_update=wl.tsmu, flags=wl.flags, out=out,
                                 selected=sel, n_selected=ns, workspace_buf=ws)

    step()
    torch.cuda.synchronize()
    want = (sel.clone(), ns.clone(), out.clone())
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            step()
    torch.cuda.current_stream().wait_stream(cs)
    for rep in range(3):
        sel.fill_(-7)
        out.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, want[0]) and torch.equal(ns, want[1]), rep
        assert torch.equal(out.view(torch.int16), want[2].view(torch.int16)), rep
        step()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want[2].view(torch.int16))
