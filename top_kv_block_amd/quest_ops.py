"""Page-3 (select_attention_operators) call shapes on top of the qsparse binding.

"ops-transformer select_attention_operators" (page 3), sections "三个核心算子" and
"quest_prefill_metadata: 元数据构建原理" / "使用示例": the torch interface there has
quest_prefill_metadata, quest_block_select_paged (allocates its output),
quest_block_select_paged_in_out (caller's output, window forcing off) and
quest_block_select_paged_in_out_w (caller's output, a host tokens_since_metadata_update
that turns sink + local-window forcing on). These wrappers give the same names and
argument orders; every call goes to the HIP library through top_kv_block_amd.qsparse.

Differences, all on purpose:
  - the page's kernel allocates [B, N, k_round] with k rounded up for 32-byte alignment
    and returns the first k columns; here the output is [B, N, k] directly (the rounding
    is a buffer-alignment detail of that hardware and changes no index);
  - k need not be a multiple of 8, and k larger than a request's block count is defined:
    the extra entries are -1 (the page reports unspecified indices there);
  - indices come back in ascending block order.
"""

from __future__ import annotations

import torch

from . import qsparse as qs

_nsel_cache = {}
_tsmu_cache = {}


def _n_selected(B, N, device):
    key = (torch.device(device).index or 0, B, N)
    t = _nsel_cache.get(key)
    if t is None:
        t = torch.empty((B, N), dtype=torch.int32, device=device)
        _nsel_cache[key] = t
    return t


def _tsmu_tensor(value, B, device):
    key = (torch.device(device).index or 0, B, int(value))
    t = _tsmu_cache.get(key)
    if t is None:
        t = torch.full((B,), int(value), dtype=torch.int32, device=device)
        _tsmu_cache[key] = t
    return t


def quest_prefill_metadata(k_cache, seq_lens, block_tables, metadata_block_tables, maxblocks, minblocks):
    """Builds the max/min metadata in place. Argument order of the page's runnable example
    (seq_lens before block_tables); its signature line lists them the other way round, and
    the order has no effect on the result."""
    qs.qs_build_metadata(k_cache, block_tables, seq_lens, metadata_block_tables, maxblocks, minblocks)


def quest_block_select_paged(query, maxblocks, minblocks, metadata_block_tables, seq_lens, k):
    """Top-k blocks per (request, KV head) by the Quest bound, no forcing. Returns [B, N, k] int32."""
    B, N = query.shape[0], maxblocks.shape[2]
    out = torch.empty((B, N, int(k)), dtype=torch.int32, device=query.device)
    qs.qs_block_select(query, maxblocks, minblocks, metadata_block_tables, seq_lens, int(k), flags=0,
                       selected=out, n_selected=_n_selected(B, N, query.device))
    return out


def quest_block_select_paged_in_out(query, maxblocks, minblocks, metadata_block_tables, seq_lens,
                                    selected_indices):
    """As quest_block_select_paged, into the caller's [B, N, k] int32 tensor."""
    B, N, k = selected_indices.shape
    qs.qs_block_select(query, maxblocks, minblocks, metadata_block_tables, seq_lens, int(k), flags=0,
                       selected=selected_indices, n_selected=_n_selected(B, N, query.device))


def quest_block_select_paged_in_out_w(query, maxblocks, minblocks, metadata_block_tables, seq_lens,
                                      tokens_since_metadata_update, selected_indices):
    """As _in_out, with the sink block and the local window forced in. tokens_since_metadata_update
    is one host int for the whole batch; -1 (any negative value) turns the forcing off."""
    B, N, k = selected_indices.shape
    ts = _tsmu_tensor(tokens_since_metadata_update, B, query.device)
    qs.qs_block_select(query, maxblocks, minblocks, metadata_block_tables, seq_lens, int(k), tokens_since_update=ts,
                       flags=qs.QS_FORCE_SINK | qs.QS_FORCE_WINDOW, selected=selected_indices,
                       n_selected=_n_selected(B, N, query.device))
