"""qs_select_attn_decode_static (the fused Quest selection + attention on the library's
static device scratch) against qs_select_attn_decode (the same call with a workspace).

Two calls in a row through the C ABI, the second smaller than the first, each bitwise
equal (output and selection) to the workspace call on the same inputs; the first uses the
scratch for the long rows' scores and the split partials, the second only for partials,
so the second also shows that the first call's leftovers do not leak into it. The checked
build's variant (its verdict word in the same array) gives the same results, and sizes
beyond the scratch are refused on the host.
"""

import pytest
import torch

from tests.conftest import gpu_available
from top_kv_block_amd import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

DEV = "cuda:0"

CASES = [
    # seed, B, H, N, BS, lens, k, dtype, flags, tsmu
    (91, 6, 32, 8, 128, [128 * 700 + 9, 128 * 300, 128 * 1000, 128 * 64 + 1, 128 * 500, 77], 64, torch.bfloat16, 3,
     [9, 0, 127, 1, 5, 0]),                                                     # long rows: scores + partials
    (92, 2, 16, 4, 64, [64 * 90 + 3, 64 * 12], 8, torch.float16, 3, [3, 0]),    # short rows: partials only
]


def _run(qs, wl, static, checked=False):
    mx = torch.zeros((wl.num_meta_blocks, wl.BS, wl.N, wl.D), dtype=wl.k_cache.dtype, device=DEV)
    mn = torch.zeros_like(mx)
    qs.qs_build_metadata(wl.k_cache, wl.block_tables, wl.meta_seq_lens, wl.meta_tables, mx, mn)
    out = torch.full((wl.B, wl.H, wl.D), 9.0, dtype=wl.query.dtype, device=DEV)
    sel = torch.full((wl.B, wl.N, wl.k), -7, dtype=torch.int32, device=DEV)
    ns = torch.full((wl.B, wl.N), -7, dtype=torch.int32, device=DEV)
    args = (wl.query, mx, mn, wl.meta_tables, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens, wl.k)
    kw = dict(tokens_since_update=wl.tsmu, flags=wl.flags, selected=sel, n_selected=ns)
    if static:
        if checked:
            with qs.checked_calls():
                qs.qs_select_attn_decode_static(*args, out, **kw)
        else:
            qs.qs_select_attn_decode_static(*args, out, **kw)
    else:
        qs.qs_select_attn_decode(*args, out=out, **kw)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu(), sel.cpu(), ns.cpu()


def test_static_scratch_matches_workspace_call_twice():
    from top_kv_block_amd import qsparse as qs
    wls = []
    for seed, B, H, N, BS, lens, k, dtype, flags, tsmu in CASES:
        wl = W.random_case(seed, B, H, N, BS, lens, k=k, dtype=dtype, flags=flags, tsmu=tsmu)
        wl.meta_seq_lens = (wl.seq_lens - wl.tsmu.clamp(min=0)).clamp(min=0)
        wls.append(wl.to(DEV))
    need = [qs.select_attn_workspace_bytes(wl.B, wl.H, wl.N, wl.BS, wl.mmbpr, wl.k, qs._dtype_code(wl.query))
            for wl in wls]
    assert need[0] > need[1] > 256, need              # the first call uses more of the scratch than the second
    for i, wl in enumerate(wls):
        print(f"[gpu-case] static scratch call {i}: B={wl.B} H={wl.H} BS={wl.BS} k={wl.k} scratch {need[i]} B",
              flush=True)
        got = _run(qs, wl, static=True)
        want = _run(qs, wl, static=False)
        for g, w in zip(got, want):
            assert torch.equal(g, w)
    # the checked build's variant keeps its verdict word in the same array
    got = _run(qs, wls[1], static=True, checked=True)
    want = _run(qs, wls[1], static=False)
    for g, w in zip(got, want):
        assert torch.equal(g, w)


def test_static_scratch_refuses_larger_sizes():
    from top_kv_block_amd import qsparse as qs
    # 1024 requests of up to 1024 blocks at k = 128 (two operations): 32 MiB of select scores
    # plus the selection, beyond the 32 MiB of scratch
    B, H, N, BS, mmbpr, k = 1024, 32, 8, 128, 8, 128
    need = qs.select_attn_workspace_bytes(B, H, N, BS, mmbpr, k, qs.QS_BF16)
    assert need > qs.QS_STATIC_SCRATCH_BYTES
    q = torch.zeros((B, H, 128), dtype=torch.bfloat16, device=DEV)
    meta = torch.zeros((1, BS, N, 128), dtype=torch.bfloat16, device=DEV)
    mt = torch.zeros((B, mmbpr), dtype=torch.int32, device=DEV)
    kv = torch.zeros((1, BS, N, 128), dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros((B, 1), dtype=torch.int32, device=DEV)
    sl = torch.zeros((B,), dtype=torch.int32, device=DEV)
    out = torch.empty((B, H, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(qs.QsError) as e:
        qs.qs_select_attn_decode_static(q, meta, meta, mt, kv, kv, bt, sl, k, out)
    assert e.value.status == qs.QS_ERR_INVALID and "static scratch" in str(e.value)
