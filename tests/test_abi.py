"""C-ABI tests that need no GPU: the library loads, exports every function the header
declares, and rejects invalid arguments on the host before any HIP call. Every test runs
against both builds (libqsparse.so and libqsparse_checked.so): the checked build's device
check comes after the host checks, so it rejects the same calls the same way.

Every invalid call below also passes B = 0 where B is not under test: B = 0 returns
before any launch, so a check that wrongly passed would still enqueue nothing.
"""

import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qsparse.h")


@pytest.fixture(scope="module", params=["plain", "checked"])
def qs(request):
    from top_kv_block_amd import qsparse
    if request.param == "plain":
        yield qsparse
    else:
        with qsparse.checked_calls():
            yield qsparse


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:qs_status|size_t|int32_t|const char\s*\*)\s*(qs_\w+)\s*\(", text, re.M)))


def test_header_declares_the_operations():
    names = _declared_functions()
    for n in ("qs_build_metadata", "qs_update_metadata", "qs_block_select", "qs_probe_select",
              "qs_sparse_attn_decode", "qs_select_attn_decode", "qs_probe_attn_decode", "qs_prefill_importance"):
        assert n in names


def test_library_exports_every_declared_symbol(qs):
    names = _declared_functions()
    assert set(names) == set(qs.EXPORTS)
    for n in names:
        assert hasattr(qs.lib, n), n
    assert qs.lib.qs_version().decode().startswith("qsparse")
    checked = qs.lib._name.endswith("libqsparse_checked.so")
    assert qs.lib.qs_checked_build() == (1 if checked else 0)
    assert ("checked" in qs.lib.qs_version().decode()) == checked


FAKE = ctypes.c_void_p(1 << 20)        # never dereferenced: every call below fails validation
WS = ctypes.c_void_p(1 << 20)          # 256-byte aligned fake workspace


def _meta(qs, **kw):
    a = dict(B=1, N=8, D=128, BS=128, dt=qs.QS_BF16, kc=FAKE, nkv=4, bt=FAKE, mkbpr=4, sl=FAKE, mt=FAKE,
             mmbpr=1, mx=FAKE, mn=FAKE, nmeta=1)
    a.update(kw)
    return qs.lib.qs_build_metadata(a["B"], a["N"], a["D"], a["BS"], a["dt"], a["kc"], a["nkv"], a["bt"],
                                    a["mkbpr"], a["sl"], a["mt"], a["mmbpr"], a["mx"], a["mn"], a["nmeta"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=64, B=0), 2), (dict(BS=100, B=0), 2), (dict(BS=256, B=0), 2), (dict(dt=2, B=0), 2),
    (dict(B=-1), 1), (dict(N=0, B=0), 1), (dict(kc=None, B=0), 1), (dict(mt=None, B=0), 1),
    (dict(mx=ctypes.c_void_p((1 << 20) + 4), B=0), 1), (dict(nkv=0, B=0), 1), (dict(mmbpr=0, B=0), 1),
])
def test_build_metadata_rejects(qs, kw, status):
    assert _meta(qs, **kw) == status
    assert qs.lib.qs_last_error().decode().startswith("qs_build_metadata")


def test_build_metadata_b0_is_noop(qs):
    assert _meta(qs, B=0) == 0
    assert qs.lib.qs_last_error().decode() == ""


def _update(qs, **kw):
    a = dict(B=0, N=8, D=128, BS=128, dt=qs.QS_BF16, kc=FAKE, nkv=4, bt=FAKE, mkbpr=4, sl=FAKE, fb=FAKE, mnew=1,
             mt=FAKE, mmbpr=1, mx=FAKE, mn=FAKE, nmeta=1)
    a.update(kw)
    return qs.lib.qs_update_metadata(a["B"], a["N"], a["D"], a["BS"], a["dt"], a["kc"], a["nkv"], a["bt"],
                                     a["mkbpr"], a["sl"], a["fb"], a["mnew"], a["mt"], a["mmbpr"], a["mx"],
                                     a["mn"], a["nmeta"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), 2), (dict(BS=100), 2), (dict(dt=2), 2), (dict(B=-1), 1), (dict(fb=None), 1),
    (dict(mnew=0), 1), (dict(mnew=-3), 1), (dict(kc=None), 1), (dict(mn=ctypes.c_void_p((1 << 20) + 8)), 1),
    (dict(nmeta=0), 1), (dict(mkbpr=0), 1),
])
def test_update_metadata_rejects(qs, kw, status):
    assert _update(qs, **kw) == status
    assert qs.lib.qs_last_error().decode().startswith("qs_update_metadata")


def test_update_metadata_b0_is_noop(qs):
    assert _update(qs) == 0
    assert qs.lib.qs_last_error().decode() == ""


def _select(qs, **kw):
    a = dict(B=0, H=32, N=8, D=128, BS=128, dt=qs.QS_BF16, q=FAKE, mx=FAKE, mn=FAKE, nmeta=1, mt=FAKE, mmbpr=1,
             sl=FAKE, ts=None, flags=0, k=8, sel=FAKE, nsel=FAKE, sc=None, ws=WS, wsb=1 << 30)
    a.update(kw)
    return qs.lib.qs_block_select(a["B"], a["H"], a["N"], a["D"], a["BS"], a["dt"], a["q"], a["mx"], a["mn"],
                                  a["nmeta"], a["mt"], a["mmbpr"], a["sl"], a["ts"], a["flags"], a["k"], a["sel"],
                                  a["nsel"], a["sc"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=30), 1), (dict(k=0), 1), (dict(flags=4), 1), (dict(flags=8), 1), (dict(dt=2), 2), (dict(D=256), 2),
    (dict(q=None), 1), (dict(ws=None), 1), (dict(ws=ctypes.c_void_p((1 << 20) + 16)), 1), (dict(wsb=16), 1),
    (dict(nsel=None), 1), (dict(mmbpr=0), 1), (dict(B=-3), 1), (dict(BS=48), 2),
])
def test_block_select_rejects(qs, kw, status):
    assert _select(qs, **kw) == status
    assert qs.lib.qs_last_error().decode().startswith("qs_block_select")


def test_block_select_workspace_size(qs):
    small = qs.block_select_workspace_bytes(20, 8, 128, 1)
    big = qs.block_select_workspace_bytes(20, 8, 128, 8)
    assert 0 < small < big and small % 256 == 0
    assert _select(qs, wsb=small) == 0                  # exactly enough, B=0: no launch


def _probe(qs, **kw):
    a = dict(B=0, H=16, N=8, D=128, BS=32, qd=qs.QS_F32, kd=qs.QS_F32, q=FAKE, kc=FAKE, nkv=128, bt=FAKE,
             mkbpr=128, sl=FAKE, imp=None, stride=0, npb=8, k=32, flags=qs.QS_RECENCY, sel=FAKE, nsel=FAKE, ps=None,
             ws=WS, wsb=1 << 30)
    a.update(kw)
    return qs.lib.qs_probe_select(a["B"], a["H"], a["N"], a["D"], a["BS"], a["qd"], a["kd"], a["q"], a["kc"],
                                  a["nkv"], a["bt"], a["mkbpr"], a["sl"], a["imp"], a["stride"], a["npb"], a["k"],
                                  a["flags"], a["sel"], a["nsel"], a["ps"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(kd=2), 2), (dict(qd=2), 2), (dict(k=0), 1), (dict(flags=1), 1), (dict(mkbpr=5000), 2),
    (dict(imp=FAKE, stride=0), 1), (dict(kc=None), 1), (dict(H=12), 1), (dict(BS=8), 2),
    (dict(ws=None), 1), (dict(ws=ctypes.c_void_p((1 << 20) + 64)), 1), (dict(wsb=16), 1),
])
def test_probe_select_rejects(qs, kw, status):
    assert _probe(qs, **kw) == status
    assert qs.lib.qs_last_error().decode().startswith("qs_probe_select")


def test_probe_select_workspace_size(qs):
    b = qs.probe_select_workspace_bytes(64, 16, 128)
    assert b == 64 * 16 * 128 * 4
    assert qs.probe_select_workspace_bytes(1, 1, 1) == 256
    assert qs.probe_select_workspace_bytes(1, 0, 1) == 0
    assert _probe(qs, wsb=qs.probe_select_workspace_bytes(0, 16, 128)) == 0


def _attn(qs, **kw):
    a = dict(B=0, H=32, N=8, D=128, BS=128, qd=qs.QS_BF16, kd=qs.QS_BF16, q=FAKE, kc=FAKE, vc=FAKE, ks=None,
             vs=None, nkv=64, bt=FAKE, mkbpr=64, sl=FAKE, sel=FAKE, nsel=FAKE, sh=8, k=16, scale=0.0, out=FAKE,
             ws=WS, wsb=1 << 30)
    a.update(kw)
    return qs.lib.qs_sparse_attn_decode(a["B"], a["H"], a["N"], a["D"], a["BS"], a["qd"], a["kd"], a["q"], a["kc"],
                                        a["vc"], a["ks"], a["vs"], a["nkv"], a["bt"], a["mkbpr"], a["sl"], a["sel"],
                                        a["nsel"], a["sh"], a["k"], a["scale"], a["out"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(sh=4), 1), (dict(sh=12), 1), (dict(sh=64), 1), (dict(k=0), 1), (dict(kd=2), 1),
    (dict(qd=2), 2), (dict(kd=7), 2), (dict(out=None), 1), (dict(wsb=8), 1), (dict(scale=float("nan")), 1),
    (dict(vc=ctypes.c_void_p((1 << 20) + 2)), 1), (dict(D=96), 2),
])
def test_sparse_attn_rejects(qs, kw, status):
    assert _attn(qs, **kw) == status
    assert qs.lib.qs_last_error().decode().startswith("qs_sparse_attn_decode")


def test_sparse_attn_workspace_size(qs):
    b = qs.sparse_attn_workspace_bytes(128, 64, 8, 128, 8, 16)
    assert b > 0 and b % 256 == 0
    assert _attn(qs, wsb=qs.sparse_attn_workspace_bytes(0, 32, 8, 128, 8, 16)) == 0
    assert qs.sparse_attn_workspace_bytes(1, 32, 8, 128, 5, 16) == 0     # H % sel_heads != 0


def _fused(qs, **kw):
    a = dict(B=0, H=32, N=8, D=128, BS=128, dt=qs.QS_BF16, q=FAKE, mx=FAKE, mn=FAKE, nmeta=1, mt=FAKE, mmbpr=1,
             kc=FAKE, vc=FAKE, nkv=64, bt=FAKE, mkbpr=64, sl=FAKE, ts=None, flags=0, k=16, scale=0.0, out=FAKE,
             sel=None, nsel=None, ws=WS, wsb=1 << 30)
    a.update(kw)
    return qs.lib.qs_select_attn_decode(a["B"], a["H"], a["N"], a["D"], a["BS"], a["dt"], a["q"], a["mx"], a["mn"],
                                        a["nmeta"], a["mt"], a["mmbpr"], a["kc"], a["vc"], a["nkv"], a["bt"],
                                        a["mkbpr"], a["sl"], a["ts"], a["flags"], a["k"], a["scale"], a["out"],
                                        a["sel"], a["nsel"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=30), 1), (dict(k=0), 1), (dict(flags=4), 1), (dict(dt=2), 2), (dict(D=64), 2), (dict(BS=48), 2),
    (dict(q=None), 1), (dict(vc=None), 1), (dict(out=None), 1), (dict(ws=None), 1), (dict(wsb=16), 1),
    (dict(ws=ctypes.c_void_p((1 << 20) + 32)), 1), (dict(sel=FAKE), 1), (dict(nsel=FAKE), 1),
    (dict(kc=ctypes.c_void_p((1 << 20) + 4)), 1), (dict(scale=float("nan")), 1), (dict(nkv=0), 1),
])
def test_select_attn_rejects(qs, kw, status):
    assert _fused(qs, **kw) == status
    assert qs.lib.qs_last_error().decode().startswith("qs_select_attn_decode")


def test_select_attn_workspace_size(qs):
    fused = qs.select_attn_workspace_bytes(128, 64, 8, 128, 2, 16, qs.QS_BF16)     # one kernel, no partials
    split = qs.select_attn_workspace_bytes(1, 4, 1, 32, 2, 8, qs.QS_F32)          # one kernel + combine
    two = qs.select_attn_workspace_bytes(8, 32, 8, 128, 8, 128, qs.QS_BF16)        # k > 64: two operations
    assert fused == 256 and split > 256 and two > 8 * 8 * 128 * 4
    assert all(x % 256 == 0 for x in (fused, split, two))
    assert qs.select_attn_workspace_bytes(1, 30, 8, 128, 1, 8, qs.QS_BF16) == 0
    assert qs.select_attn_workspace_bytes(1, 32, 8, 128, 1, 8, qs.QS_I8) == 0
    assert _fused(qs, sel=FAKE, nsel=FAKE) == 0


def _pattn(qs, **kw):
    a = dict(B=0, H=16, N=8, D=128, BS=32, qd=qs.QS_F32, kd=qs.QS_F32, q=FAKE, kc=FAKE, vc=FAKE, ks=None, vs=None,
             pk=None, pkd=qs.QS_F32, nkv=128, bt=FAKE, mkbpr=128, sl=FAKE, imp=None, stride=0, npb=8, k=32,
             flags=qs.QS_RECENCY, scale=0.0, out=FAKE, sel=None, nsel=None, ws=WS, wsb=1 << 30)
    a.update(kw)
    return qs.lib.qs_probe_attn_decode(a["B"], a["H"], a["N"], a["D"], a["BS"], a["qd"], a["kd"], a["q"], a["kc"],
                                       a["vc"], a["ks"], a["vs"], a["pk"], a["pkd"], a["nkv"], a["bt"], a["mkbpr"],
                                       a["sl"], a["imp"], a["stride"], a["npb"], a["k"], a["flags"], a["scale"],
                                       a["out"], a["sel"], a["nsel"], a["ws"], a["wsb"], None)


Q8 = dict(kd=2, ks=FAKE, vs=FAKE, pk=FAKE)            # a valid int8-cache argument set


@pytest.mark.parametrize("kw,status", [
    (dict(kd=2), 1), (dict(Q8, ks=None), 1), (dict(Q8, vs=None), 1), (dict(Q8, pk=None), 1),
    (dict(Q8, pkd=2), 2), (dict(Q8, pk=ctypes.c_void_p((1 << 20) + 8)), 1), (dict(ks=FAKE), 1), (dict(pk=FAKE), 1),
    (dict(qd=2), 2), (dict(k=0), 1), (dict(k=4097), 1), (dict(flags=1), 1), (dict(mkbpr=5000), 2),
    (dict(imp=FAKE, stride=0), 1), (dict(vc=None), 1), (dict(out=None), 1), (dict(sel=FAKE), 1),
    (dict(nsel=FAKE), 1), (dict(H=12), 1), (dict(BS=8), 2), (dict(D=96), 2), (dict(ws=None), 1),
    (dict(ws=ctypes.c_void_p((1 << 20) + 64)), 1), (dict(wsb=16), 1), (dict(scale=float("nan")), 1),
    (dict(kc=ctypes.c_void_p((1 << 20) + 4)), 1),
])
def test_probe_attn_rejects(qs, kw, status):
    assert _pattn(qs, **kw) == status
    assert qs.lib.qs_last_error().decode().startswith("qs_probe_attn_decode")


def test_probe_attn_workspace_size(qs):
    # the probe keys (B * H * mkbpr uint32), then the attention partials: 16 rows of one
    # query head want 2048 / 16 = 128 slot splits, capped at k = 32, each a (D + 2)-float record
    assert qs.probe_attn_workspace_bytes(1, 16, 8, 128, 32) == 16 * 128 * 4 + 16 * 32 * 130 * 4
    # 2048 rows: one split each, no partials
    assert qs.probe_attn_workspace_bytes(64, 32, 8, 100, 8) == 64 * 32 * 100 * 4
    assert qs.probe_attn_workspace_bytes(1, 12, 8, 128, 32) == 0
    assert _pattn(qs, wsb=qs.probe_attn_workspace_bytes(0, 16, 8, 128, 32)) == 0
    assert _pattn(qs, **Q8) == 0                     # an int8 cache with its scales and probe K is accepted


def _imp(qs, **kw):
    a = dict(B=0, H=16, N=8, D=128, BS=32, dt=qs.QS_F32, q=FAKE, ml=4096, kc=FAKE, nkv=128, bt=FAKE, mkbpr=128,
             sl=FAKE, scale=0.0, imp=FAKE, stride=4096, himp=None, ws=WS, wsb=1 << 30)
    a.update(kw)
    return qs.lib.qs_prefill_importance(a["B"], a["H"], a["N"], a["D"], a["BS"], a["dt"], a["q"], a["ml"], a["kc"],
                                        a["nkv"], a["bt"], a["mkbpr"], a["sl"], a["scale"], a["imp"], a["stride"],
                                        a["himp"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=2), 2), (dict(D=64), 2), (dict(H=12), 1), (dict(q=None), 1), (dict(imp=None), 1),
    (dict(ws=None), 1), (dict(wsb=16), 1), (dict(ml=-1), 1), (dict(stride=0), 1), (dict(nkv=0), 1),
    (dict(kc=ctypes.c_void_p((1 << 20) + 8)), 1), (dict(scale=float("nan")), 1), (dict(BS=24), 2),
])
def test_prefill_importance_rejects(qs, kw, status):
    assert _imp(qs, **kw) == status
    assert qs.lib.qs_last_error().decode().startswith("qs_prefill_importance")


def test_prefill_importance_workspace_size(qs):
    # the minimum: fp32 row normalisers + per chunk (row max, row sum, column sums), for the
    # larger of the two splits (fp32: one chunk; 16-bit: tiles of 128 rows, chunked below
    # 8192 x 64 rows x heads x requests): 4096 rows x 16 heads -> 8 chunks; 2 x 32 heads x
    # 8192 rows -> 1; then the fp32 path's stored scores, T (T + 1) / 2 blocks of 16 x 16
    # floats per (request, head) with T = ceil(max_len / 16), when they take at most 2 GiB
    def blocks(max_len):
        t = -(-max_len // 16)
        return t * (t + 1) // 2
    base = (1 + 3 * 8) * 16 * 4096 * 4
    assert qs.prefill_importance_workspace_bytes(1, 16, 4096) == base + 16 * blocks(4096) * 1024
    # 2 x 32 heads x 8192 rows: 8.6 GB of scores, over the cap: the minimum only
    assert qs.prefill_importance_workspace_bytes(2, 32, 8192) == (1 + 3 * 1) * 2 * 32 * 8192 * 4
    # (1 + 3 * 1 chunk) * 100 * 4 = 1600, rounded up to 256 B, then 7 * 8 / 2 blocks
    assert qs.prefill_importance_workspace_bytes(1, 1, 100) == 1792 + blocks(100) * 1024
    assert qs.prefill_importance_workspace_bytes(0, 16, 4096) == 256
    assert qs.prefill_importance_workspace_bytes(1, 0, 4096) == 0
    assert _imp(qs, imp=None, himp=FAKE, wsb=qs.prefill_importance_workspace_bytes(0, 16, 4096)) == 0
    # what a call requires is the minimum (without the scores, which it then recomputes):
    # one byte less is refused before anything is launched, naming the minimum
    assert _imp(qs, B=1, imp=None, himp=FAKE, wsb=base - 1) == 1
    assert qs.lib.qs_last_error().decode().endswith(f"{base - 1} bytes, {base} needed")
    # the binding asks for the full size for fp32 inputs and the minimum for 16-bit ones
    # (which never store their scores)
    assert qs.prefill_importance_call_workspace_bytes(1, 16, 4096, True) == base + 16 * blocks(4096) * 1024
    assert qs.prefill_importance_call_workspace_bytes(1, 16, 4096, False) == base
    assert qs.prefill_importance_call_workspace_bytes(1, 1, 100, False) == 1792
    big = (1 + 3 * 1) * 2 * 32 * 8192 * 4
    assert qs.prefill_importance_call_workspace_bytes(2, 32, 8192, False) == big
    assert qs.prefill_importance_call_workspace_bytes(2, 32, 8192, True) == big
    assert qs.prefill_importance_call_workspace_bytes(0, 16, 4096, False) == 256
    assert qs.prefill_importance_call_workspace_bytes(1, 0, 4096, False) == 0


def test_binding_refuses_cpu_tensors(qs):
    import torch
    x = torch.zeros((1, 4, 128))
    with pytest.raises(ValueError):
        qs.qs_sparse_attn_decode(x, torch.zeros((1, 32, 1, 128)), torch.zeros((1, 32, 1, 128)),
                                 torch.zeros((1, 1), dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
                                 torch.zeros((1, 1, 1), dtype=torch.int32), torch.zeros((1, 1), dtype=torch.int32))


def test_page3_wrappers_exist_and_refuse_cpu_tensors(qs):
    import torch
    from top_kv_block_amd import quest_ops as Q
    for name in ("quest_prefill_metadata", "quest_block_select_paged", "quest_block_select_paged_in_out",
                 "quest_block_select_paged_in_out_w"):
        assert callable(getattr(Q, name))
    q = torch.zeros((1, 8, 128), dtype=torch.float16)
    m = torch.zeros((1, 128, 2, 128), dtype=torch.float16)
    t = torch.zeros((1, 1), dtype=torch.int32)
    with pytest.raises(ValueError):
        Q.quest_block_select_paged(q, m, m, t, torch.ones(1, dtype=torch.int32), 4)


def test_workspace_size_queries_follow_the_loaded_library(qs):
    """The binding remembers workspace-size answers per loaded library: under both builds
    (and after switching between them) every query equals a direct call of the library."""
    cases = [("select_attn_workspace_bytes", "qs_select_attn_workspace_bytes", (8, 32, 8, 128, 8, 64, qs.QS_BF16)),
             ("block_select_workspace_bytes", "qs_block_select_workspace_bytes", (20, 8, 128, 1)),
             ("probe_select_workspace_bytes", "qs_probe_select_workspace_bytes", (1, 16, 128)),
             ("sparse_attn_workspace_bytes", "qs_sparse_attn_workspace_bytes", (1, 16, 8, 128, 16, 32)),
             ("probe_attn_workspace_bytes", "qs_probe_attn_workspace_bytes", (1, 16, 8, 128, 32)),
             ("prefill_importance_workspace_bytes", "qs_prefill_importance_workspace_bytes", (1, 16, 4096))]
    for _ in range(2):  # the second pass answers from the remembered values
        for wrapper, fn, args in cases:
            assert getattr(qs, wrapper)(*args) == getattr(qs.lib, fn)(*args), wrapper
