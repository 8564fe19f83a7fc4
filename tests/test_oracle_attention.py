"""Oracle pins for exact attention over the selected blocks.

Pinned against: torch's scaled_dot_product_attention in float64 on the CPU when every
block is selected (dense attention) or on the gathered selected tokens, the
single-token closed form, order invariance, the convex-hull property, the int8 path on
exactly representable queries, and hand-picked quantiser cases.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from top_kv_block_amd import workloads as W
from tests.helpers import cdiv, f64, request_tokens


def _sdpa(q, k, v, scale):
    """Library attention: q [D], k/v [T, D] float64 numpy -> [D]."""
    qt = torch.from_numpy(q)[None, None, None, :]
    kt = torch.from_numpy(k)[None, None]
    vt = torch.from_numpy(v)[None, None]
    return F.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, 0, 0].numpy()


def _all_blocks(wl):
    nbmax = wl.block_tables.shape[1]
    rows = wl.sel_heads
    sel = torch.arange(nbmax, dtype=torch.int32).repeat(wl.B, rows, 1)
    ns = torch.full((wl.B, rows), nbmax, dtype=torch.int32)
    return sel, ns


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_all_blocks_selected_is_dense_attention(oracle, dtype):
    lens = [3 * 32 + 11, 5 * 32, 1]
    wl = W.random_case(41, 3, 8, 2, 32, lens, k=8, dtype=dtype)
    sel, ns = _all_blocks(wl)
    out = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens,
                                    sel, ns, wl.N)
    scale = 1.0 / np.sqrt(wl.D)
    for b in range(wl.B):
        K, V = request_tokens(wl, b, "k"), request_tokens(wl, b, "v")
        for h in range(wl.H):
            kh = h // wl.G
            want = _sdpa(f64(wl.query[b, h]), K[:, kh], V[:, kh], scale)
            np.testing.assert_allclose(out[b, h], want, rtol=1e-10, atol=1e-12)


def test_selected_subset_is_attention_on_gathered_tokens(oracle):
    lens = [20 * 32 + 3]
    wl = W.random_case(42, 1, 16, 8, 32, lens, k=4, sel_heads=16)
    g = torch.Generator().manual_seed(1)
    sel = torch.stack([torch.randperm(21, generator=g)[:4] for _ in range(16)]).to(torch.int32)[None]
    sel[0, 3] = torch.tensor([20, 0, 5, 9], dtype=torch.int32)       # includes the partial block
    ns = torch.full((1, 16), 4, dtype=torch.int32)
    out = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens,
                                    sel, ns, 16, softmax_scale=0.3)
    K, V = request_tokens(wl, 0, "k"), request_tokens(wl, 0, "v")
    for h in range(16):
        toks = np.concatenate([np.arange(32 * i, min(32 * (i + 1), lens[0])) for i in sel[0, h].tolist()])
        kh = h // 2
        want = _sdpa(f64(wl.query[0, h]), K[toks, kh], V[toks, kh], 0.3)
        np.testing.assert_allclose(out[0, h], want, rtol=1e-10, atol=1e-12)


def test_single_token_selection_returns_v(oracle):
    L = 4 * 32 + 1
    wl = W.random_case(43, 1, 4, 2, 32, [L], k=2)
    sel = torch.tensor([[[4, -1], [4, -1]]], dtype=torch.int32)
    ns = torch.tensor([[1, 1]], dtype=torch.int32)
    out = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens,
                                    sel, ns, 2)
    V = request_tokens(wl, 0, "v")
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], V[L - 1, h // 2])


def test_order_invariance_invalid_entries_and_hull(oracle):
    L = 9 * 32
    wl = W.random_case(44, 1, 4, 1, 32, [L], k=5)
    a = torch.tensor([[[1, 4, 7, -1, -1]]], dtype=torch.int32)
    b = torch.tensor([[[7, 1, 4, 100, -1]]], dtype=torch.int32)           # shuffled + out of range
    oa = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens,
                                   a, torch.tensor([[3]], dtype=torch.int32), 1)
    ob = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens,
                                   b, torch.tensor([[5]], dtype=torch.int32), 1)
    np.testing.assert_allclose(oa, ob, rtol=1e-13, atol=1e-15)
    V = request_tokens(wl, 0, "v")[:, 0]
    toks = np.concatenate([np.arange(32 * i, 32 * (i + 1)) for i in (1, 4, 7)])
    lo, hi = V[toks].min(axis=0), V[toks].max(axis=0)
    assert np.all(oa[0] >= lo - 1e-12) and np.all(oa[0] <= hi + 1e-12)


def test_empty_selection_gives_zero(oracle):
    wl = W.random_case(45, 2, 2, 1, 32, [0, 64], k=2)
    sel = torch.tensor([[[-1, -1]], [[-1, 5]]], dtype=torch.int32)
    out = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens,
                                    sel, torch.tensor([[0], [2]], dtype=torch.int32), 1)
    assert np.all(out == 0.0)


def test_int8_exact_query_matches_dequantized_attention(oracle):
    """Query entries are integer multiples of 2^-6 with |max| = 127 * 2^-6: its
    absmax/127 scale and codes are exact, so int8 attention must equal float64
    attention on the dequantised K and V."""
    L = 6 * 32 + 13
    wl = W.random_case(46, 1, 4, 2, 32, [L], k=4, int8=True)
    g = torch.Generator().manual_seed(3)
    codes = torch.randint(-127, 128, (1, 4, 128), generator=g).float()
    codes[..., 0] = 127.0
    q = codes * 2.0 ** -6
    sel = torch.tensor([[[0, 2, 6, -1], [1, 3, 5, 6]]], dtype=torch.int32)
    ns = torch.tensor([[3, 4]], dtype=torch.int32)
    out = oracle.sparse_attn_decode(q, wl.k_i8, wl.v_i8, wl.block_tables, wl.seq_lens, sel, ns, 2,
                                    k_scale=wl.k_scale, v_scale=wl.v_scale)
    nb = cdiv(L, 32)
    phys = wl.block_tables[0, :nb].long()
    Kd = (wl.k_i8[phys].double() * wl.k_scale[phys].double()[..., None]).reshape(-1, 2, 128)[:L].numpy()
    Vd = (wl.v_i8[phys].double() * wl.v_scale[phys].double()[..., None]).reshape(-1, 2, 128)[:L].numpy()
    for h in range(4):
        blocks = sel[0, h // 2, :ns[0, h // 2]].tolist()
        toks = np.concatenate([np.arange(32 * i, min(32 * (i + 1), L)) for i in blocks])
        want = _sdpa(f64(q[0, h]), Kd[toks, h // 2], Vd[toks, h // 2], 1 / np.sqrt(128))
        np.testing.assert_allclose(out[0, h], want, rtol=1e-12, atol=1e-13)


def test_query_quantiser_cases(oracle):
    s = 2.0 ** -4                      # scale = absmax / 127 with absmax = 127 * s
    row = np.zeros(128, np.float32)
    row[0] = 127 * s
    row[1:9] = np.array([2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 126.5, -0.5], np.float32) * s
    codes, scale = oracle.quantize_row_i8(row)
    assert scale == np.float32(s)
    assert codes[:9].tolist() == [127, 2, 4, -2, -4, 0, 2, 126, 0]     # half to even
    codes, scale = oracle.quantize_row_i8(np.zeros(128, np.float32))
    assert scale == 0.0 and not codes.any()


def test_bf16_is_exact_widening(oracle):
    wl = W.random_case(47, 1, 4, 2, 32, [150], k=3, dtype=torch.bfloat16)
    sel = torch.tensor([[[0, 2, 4], [1, 3, 4]]], dtype=torch.int32)
    ns = torch.tensor([[3, 3]], dtype=torch.int32)
    a = oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, sel, ns, 2)
    b = oracle.sparse_attn_decode(wl.query.float(), wl.k_cache.float(), wl.v_cache.float(), wl.block_tables,
                                  wl.seq_lens, sel, ns, 2)
    assert np.array_equal(a, b)


def test_widening_matches_library_decoders(oracle):
    """Every stored element the oracle reads is widened exactly: all 65536 binary16 and
    bfloat16 bit patterns against numpy's and torch's own conversions, and int8."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = bits.view(np.float16)
    got = oracle.widen(h)
    want = h.astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))      # -0 stays -0
    bf = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    got = oracle.widen(bf)
    want = bf.float().double().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan], want[~nan])
    i8 = np.arange(-128, 128, dtype=np.int8)
    assert np.array_equal(oracle.widen(i8), i8.astype(np.float64))
