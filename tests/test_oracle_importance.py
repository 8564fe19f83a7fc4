"""Oracle pins for the prefill importance (page 1, section 1, signal 2: the attention
the prefill gave each token, summed over the rows that saw it and over heads).

Pinned against: torch.softmax of the causally masked float64 score matrix (library
routine), the row-mass identity (each query row's weights sum to 1, so the importance
sums to H * L), the harmonic-number closed form when every key is equal, the single-token
case, and head-range additivity.
"""

import math

import numpy as np
import pytest
import torch

from top_kv_block_amd import workloads as W
from tests.helpers import f64, request_tokens


def _torch_head_imp(wl, q, b, h, scale):
    L = int(wl.seq_lens[b])
    K = request_tokens(wl, b, "k")[:, h // wl.G]                 # [L, D] float64
    Q = f64(q[b, :L, h])
    S = torch.from_numpy(scale * (Q @ K.T))
    S = S.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), diagonal=1), float("-inf"))
    return torch.softmax(S, dim=1).sum(dim=0).numpy()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_matches_causal_softmax(oracle, dtype):
    wl = W.random_case(91, 2, 4, 2, 16, [37, 50], k=2, dtype=dtype, with_v=False)
    q = W.prefill_queries(wl, 1)
    imp, himp = oracle.prefill_importance(q, wl.k_cache, wl.block_tables, wl.seq_lens, wl.N, stride=64)
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        tot = np.zeros(L)
        for h in range(wl.H):
            want = _torch_head_imp(wl, q, b, h, 1.0 / math.sqrt(wl.D))
            np.testing.assert_allclose(himp[b, h, :L], want, rtol=1e-12, atol=1e-12)
            tot += want
        np.testing.assert_allclose(imp[b, :L], tot, rtol=1e-12, atol=1e-12)
        assert not imp[b, L:].any() and not himp[b, :, L:].any()


def test_row_mass_and_scale(oracle):
    wl = W.random_case(92, 3, 8, 4, 32, [100, 1, 65], k=2, with_v=False)
    q = W.prefill_queries(wl, 2)
    for scale in (0.0, 0.3):
        imp, himp = oracle.prefill_importance(q, wl.k_cache, wl.block_tables, wl.seq_lens, wl.N, softmax_scale=scale)
        for b in range(wl.B):
            L = int(wl.seq_lens[b])
            assert abs(imp[b].sum() - wl.H * L) <= 1e-9 * wl.H * L
            # the first token is seen by every row; the last one only by itself
            np.testing.assert_allclose(himp[b, :, L - 1].sum(), imp[b, L - 1], rtol=1e-12)
            assert np.all(himp[b, :, :L] <= np.arange(L, 0, -1)[None, :] + 1e-12)


def test_identical_keys_give_harmonic_tail(oracle):
    """Equal keys: row t spreads 1/(t+1) over tokens 0..t, so imp[s] = H_L - H_s per head."""
    wl = W.random_case(93, 1, 4, 2, 16, [70], k=2, with_v=False)
    kc = wl.k_cache.clone()
    kc[:] = kc[0, 0]
    q = W.prefill_queries(wl, 3)
    imp, himp = oracle.prefill_importance(q, kc, wl.block_tables, wl.seq_lens, wl.N)
    L = 70
    harm = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, L + 1))])
    want = harm[L] - harm[np.arange(L)]
    for h in range(wl.H):
        np.testing.assert_allclose(himp[0, h, :L], want, rtol=1e-12)


def test_single_token_and_empty(oracle):
    wl = W.random_case(94, 2, 6, 3, 16, [1, 0], k=1, with_v=False)
    q = W.prefill_queries(wl, 4, max_len=4)
    imp, himp = oracle.prefill_importance(q, wl.k_cache, wl.block_tables, wl.seq_lens, wl.N)
    assert imp[0, 0] == 6.0 and not imp[0, 1:].any() and not imp[1].any()


def test_head_range_is_additive(oracle):
    wl = W.random_case(95, 1, 8, 2, 16, [90], k=2, with_v=False)
    q = W.prefill_queries(wl, 5)
    full, fh = oracle.prefill_importance(q, wl.k_cache, wl.block_tables, wl.seq_lens, wl.N)
    part, ph = oracle.prefill_importance(q, wl.k_cache, wl.block_tables, wl.seq_lens, wl.N, heads=(2, 5))
    np.testing.assert_array_equal(ph[:, 2:5], fh[:, 2:5])
    assert not ph[:, :2].any() and not ph[:, 5:].any()
    np.testing.assert_allclose(part[0], fh[0, 2:5].sum(axis=0), rtol=1e-13)
