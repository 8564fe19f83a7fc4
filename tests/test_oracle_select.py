"""Oracle pins for the Quest block selection (page 3's grouped-query upper-bound score,
top-k with lower-index ties, sink/window forcing).

Pinned against: the Quest upper bound checked with numpy dot products, closed forms
(single-key metadata, non-negative query, absent blocks), the GQA mean on exactly
representable queries, numpy.lexsort as the ordering, brute force over subsets, and
the tiny workload's planted needle.
"""

import itertools

import numpy as np
import pytest
import torch

from top_kv_block_amd import workloads as W
from tests.helpers import as_sets, cdiv, check_selection_rows, f64, golden_rows


def _build(oracle, wl):
    return oracle.build_metadata(wl.k_cache, wl.block_tables, wl.meta_seq_lens, wl.meta_tables,
                                 wl.num_meta_blocks)


def _group_equal_query(wl, seed=0):
    """Make every query head of a group equal to its group's first head, so the grouped
    query is known without computing a mean."""
    q = wl.query.clone()
    G = wl.G
    for n in range(wl.N):
        q[:, n * G:(n + 1) * G] = q[:, n * G:n * G + 1]
    wl.query = q
    return wl


def test_quest_upper_bound(oracle):
    lens = [5 * 32 + 9, 64, 300]
    wl = _group_equal_query(W.random_case(21, 3, 8, 2, 32, lens, k=4, dtype=torch.float32))
    mx, mn = _build(oracle, wl)
    _, _, sc = oracle.block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, 4)
    for b, L in enumerate(lens):
        for n in range(wl.N):
            gq = f64(wl.query[b, n * wl.G])
            for i in range(cdiv(L, 32)):
                phys = int(wl.block_tables[b, i])
                keys = f64(wl.k_cache[phys, :min(32, L - 32 * i), n])
                dots = keys @ gq
                margin = 1e-9 * np.sum(np.abs(gq) * np.abs(keys), axis=1).max()
                assert sc[b, n, i] >= dots.max() - margin


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_single_key_metadata_is_dot(oracle, dtype):
    """max == min == k  =>  score = gq . k exactly."""
    B, H, N, D, BS = 2, 8, 4, 128, 16
    g = torch.Generator().manual_seed(5)
    keys = torch.randn((2, BS, N, D), generator=g).to(dtype)
    q = torch.randn((B, H, D), generator=g).to(dtype)
    for n in range(N):
        q[:, n * 2:(n + 1) * 2] = q[:, n * 2:n * 2 + 1]
    mt = torch.tensor([[0], [1]], dtype=torch.int32)
    sl = torch.tensor([BS * BS, 7 * BS], dtype=torch.int32)
    _, _, sc = oracle.block_select(q, keys, keys, mt, sl, 3)
    for b in range(B):
        nb = cdiv(int(sl[b]), BS)
        for n in range(N):
            want = f64(keys[b, :nb, n]) @ f64(q[b, 2 * n])
            np.testing.assert_allclose(sc[b, n, :nb], want, rtol=1e-12, atol=1e-12)


def test_nonnegative_query_scores_kmax(oracle):
    wl = W.random_case(22, 2, 4, 2, 32, [200, 64], k=3, dtype=torch.float32)
    wl.query = wl.query.abs()
    wl = _group_equal_query(wl)
    mx, mn = _build(oracle, wl)
    _, _, sc = oracle.block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, 3)
    for b in range(2):
        for n in range(2):
            gq = f64(wl.query[b, n * 2])
            for i in range(cdiv(int(wl.seq_lens[b]), 32)):
                m = int(wl.meta_tables[b, i // 32])
                np.testing.assert_allclose(sc[b, n, i], f64(mx[m, i % 32, n]) @ gq, rtol=1e-12)


def test_grouped_query_is_mean_of_contiguous_group(oracle):
    """Heads of group n are v_n + c_g * w_n with sum(c) = 0 (dyadic values, exact in
    double): the grouped query must be v_n, and group n must own heads nG..nG+G-1."""
    B, N, G, D, BS = 1, 3, 4, 128, 16
    H = N * G
    g = torch.Generator().manual_seed(9)
    v = torch.round(torch.randn((N, D), generator=g) * 64) / 64
    w = torch.round(torch.randn((N, D), generator=g) * 64) / 64
    c = torch.tensor([1.0, -1.0, 2.0, -2.0])
    q = (v[:, None, :] + c[None, :, None] * w[:, None, :]).reshape(1, H, D)
    keys = torch.randn((1, BS, N, D), generator=g)
    mt = torch.zeros((1, 1), dtype=torch.int32)
    sl = torch.tensor([BS * BS], dtype=torch.int32)
    _, _, sc = oracle.block_select(q, keys, keys, mt, sl, 2)
    for n in range(N):
        np.testing.assert_allclose(sc[0, n, :BS], f64(keys[0, :, n]) @ f64(v[n]), rtol=1e-12, atol=1e-12)


def test_absent_metadata_scores_zero(oracle):
    B, H, N, D, BS = 1, 2, 1, 128, 16
    q = torch.randn((B, H, D))
    z = torch.zeros((1, BS, N, D))
    _, _, sc = oracle.block_select(q, z, z, torch.zeros((1, 1), dtype=torch.int32),
                                   torch.tensor([5 * BS], dtype=torch.int32), 2)
    assert np.all(sc[0, 0, :5] == 0.0)


@pytest.mark.parametrize("k", [1, 3, 8, 40, 200])
def test_selection_is_lexsort_topk(oracle, k):
    lens = [1000, 37, 0, 64 * 32]
    wl = W.random_case(23, 4, 8, 4, 32, lens, k=k, dtype=torch.bfloat16)
    mx, mn = _build(oracle, wl)
    sel, ns, sc = oracle.block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, k)
    check_selection_rows(sel, ns, k)
    for b, L in enumerate(lens):
        nb = cdiv(L, 32)
        for n in range(wl.N):
            s = sc[b, n, :nb]
            order = np.lexsort((np.arange(nb), -s))          # score desc, index asc
            want = np.sort(order[:min(k, nb)])
            assert int(ns[b, n]) == min(k, nb)
            np.testing.assert_array_equal(sel[b, n, :ns[b, n]], want)


def test_selection_bruteforce_with_ties(oracle):
    """Tiny cases with many exact ties: the selected set is the unique k-set in which
    every selected (score, -index) beats every unselected one."""
    rng = np.random.default_rng(0)
    BS, D = 16, 128
    for trial in range(30):
        nb = int(rng.integers(1, 11))
        k = int(rng.integers(1, 12))
        # few distinct channel values -> many equal scores
        vals = rng.integers(-2, 3, size=(nb, 1, 1, D)).astype(np.float32)
        meta = np.zeros((1, BS, 1, D), np.float32)
        meta[0, :nb] = vals[:, 0]
        q = torch.ones((1, 1, D))
        sel, ns, sc = oracle.block_select(q, torch.from_numpy(meta), torch.from_numpy(meta),
                                          torch.zeros((1, 1), dtype=torch.int32),
                                          torch.tensor([nb * BS - int(rng.integers(0, BS))], dtype=torch.int32), k)
        s = sc[0, 0, :nb]
        want = None
        for combo in itertools.combinations(range(nb), min(k, nb)):
            cs = set(combo)
            ok = all((s[a] > s[c]) or (s[a] == s[c] and a < c)
                     for a in cs for c in range(nb) if c not in cs)
            if ok:
                assert want is None, "ordering must single out one set"
                want = cs
        assert as_sets(sel, ns)[0] == want


def test_ties_go_to_lower_index(oracle):
    BS, D = 16, 128
    meta = torch.ones((1, BS, 1, D))
    sel, ns, _ = oracle.block_select(torch.ones((1, 2, D)), meta, meta,
                                     torch.zeros((1, 1), dtype=torch.int32),
                                     torch.tensor([12 * BS], dtype=torch.int32), 5)
    assert list(sel[0, 0]) == [0, 1, 2, 3, 4]


def test_k_at_least_blocks_returns_all(oracle):
    wl = W.random_case(24, 1, 2, 1, 32, [5 * 32 - 3], k=9, dtype=torch.float32)
    mx, mn = _build(oracle, wl)
    sel, ns, _ = oracle.block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, 9)
    assert list(sel[0, 0]) == [0, 1, 2, 3, 4, -1, -1, -1, -1] and int(ns[0, 0]) == 5


def _forced_case(oracle, L, tsmu, k, flags, cover=None, seed=25):
    BS = 32
    wl = W.random_case(seed, 1, 4, 2, BS, [L], k=k, dtype=torch.float32,
                       meta_cover=[cover if cover is not None else L], tsmu=[tsmu], flags=flags)
    mx, mn = _build(oracle, wl)
    return wl, oracle.block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, k,
                                   tsmu=wl.tsmu, flags=flags)


def test_sink_and_window_forced(oracle):
    L = 40 * 32 + 10
    nb = cdiv(L, 32)
    wl, (sel, ns, sc) = _forced_case(oracle, L, 10, 6, W.FORCE_SINK | W.FORCE_WINDOW, cover=L - 10)
    for n in range(wl.N):
        s = set(sel[0, n, :ns[0, n]].tolist())
        assert {0, nb - 1} <= s and len(s) == 6
        # the rest is the lexsort top-4 of the non-forced candidates
        cand = [i for i in range(nb) if i not in (0, nb - 1)]
        order = sorted(cand, key=lambda i: (-sc[0, n, i], i))
        assert s - {0, nb - 1} == set(order[:4])
        assert np.isnan(sc[0, n, 0]) and np.isnan(sc[0, n, nb - 1])


def test_stale_blocks_forced_then_priority(oracle):
    BS = 32
    L = 50 * BS
    # 3 full blocks decoded since the last update: blocks 47, 48, 49 lack metadata
    wl, (sel, ns, _) = _forced_case(oracle, L, 3 * BS, 8, W.FORCE_SINK | W.FORCE_WINDOW, cover=L - 3 * BS)
    for n in range(wl.N):
        assert {0, 47, 48, 49} <= set(sel[0, n, :ns[0, n]].tolist())
    # forced set larger than k: last block first, then descending, sink last
    wl, (sel, ns, _) = _forced_case(oracle, L, 3 * BS, 2, W.FORCE_SINK | W.FORCE_WINDOW, cover=L - 3 * BS)
    assert sel[0, 0].tolist() == [48, 49]
    wl, (sel, ns, _) = _forced_case(oracle, L, 3 * BS, 4, W.FORCE_SINK | W.FORCE_WINDOW, cover=L - 3 * BS)
    assert sel[0, 0].tolist() == [0, 47, 48, 49]


def test_negative_tsmu_disables_forcing(oracle):
    L = 20 * 32
    wl, (sel, ns, sc) = _forced_case(oracle, L, -1, 3, W.FORCE_SINK | W.FORCE_WINDOW)
    for n in range(wl.N):
        order = sorted(range(20), key=lambda i: (-sc[0, n, i], i))
        assert set(sel[0, n, :3].tolist()) == set(order[:3])
        assert not np.isnan(sc[0, n, :20]).any()


def test_window_only_when_aligned_is_last_block(oracle):
    L = 20 * 32
    wl, (sel, ns, sc) = _forced_case(oracle, L, 0, 3, W.FORCE_WINDOW)
    for n in range(wl.N):
        assert 19 in set(sel[0, n, :3].tolist())
        assert np.isnan(sc[0, n, 19]) and not np.isnan(sc[0, n, :19]).any()


def test_tiny_needle_selected(oracle):
    (tok, bs, want_block), = [tuple(int(x) for x in r) for r in golden_rows("tiny_needle.txt")]
    wl = W.tiny_needle()
    assert tok // bs == want_block and wl.BS == bs
    mx, mn = _build(oracle, wl)
    sel, ns, sc = oracle.block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, wl.k)
    assert want_block in set(sel[0, 0, :ns[0, 0]].tolist())


def test_oracle_deterministic(oracle):
    wl = W.random_case(26, 2, 8, 2, 32, [900, 333], k=5, dtype=torch.bfloat16)
    mx, mn = _build(oracle, wl)
    a = oracle.block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, 5)
    b = oracle.block_select(wl.query, mx, mn, wl.meta_tables, wl.seq_lens, 5)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
