"""The checked build (libqsparse_checked.so) on the GPU.

On valid inputs every call gives bitwise what the plain build gives. With sequence lengths
or table entries planted out of range it refuses exactly the calls the oracle refuses (the
oracle returns "invalid input" whenever it would have to follow an entry out of range),
names the first bad entry (lowest request first) and writes no output. Two calls check
more than the oracle needs and are only held to "every call the oracle refuses is
refused": Quest selection with forcing (the forced blocks' metadata entries are checked
too) and the fused Quest call (every block's block_tables entry is checked, selected or
not). Every planted entry is one that the plain build's kernels skip, so no run here
reads out of bounds even if a check were missing.
"""

import sys

import pytest
import torch

from tests.conftest import gpu_available
from top_kv_block_amd import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

DEV = "cuda:0"
SENT = 7.0


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def qs():
    from top_kv_block_amd import qsparse
    return qsparse


def nbs(sl, BS):
    return [max(0, -(-int(L) // BS)) for L in sl.tolist()]


# ------------------------------------------------------------------------------------------
# planted inputs: each returns the mutated (bt, sl, mt) and the message fragment that names
# the first bad entry (None when the planted entry is one no call uses)
# ------------------------------------------------------------------------------------------

def mutate(kind, wl):
    bt, sl, mt = wl.block_tables.clone(), wl.seq_lens.clone(), wl.meta_tables.clone()
    nkv, BS, nmeta = wl.k_cache.shape[0], wl.BS, wl.num_meta_blocks
    nb = nbs(sl, BS)
    last = max(b for b in range(wl.B) if nb[b] > 0)
    frag = None
    if kind == "valid":
        pass
    elif kind == "bt_last_block":
        bt[last, nb[last] - 1] = nkv
        frag = f"block_tables[{last}][{nb[last] - 1}] = {nkv} "
    elif kind == "bt_negative":
        bt[0, 0] = -7
        frag = "block_tables[0][0] = -7 "
    elif kind == "bt_past_length":          # a slot past the request's blocks: never used
        b = next(b for b in range(wl.B) if nb[b] < bt.shape[1])
        bt[b, nb[b]] = nkv + 9
    elif kind == "two_requests":            # the lower request is named
        bt[2, 1] = nkv
        bt[1, 0] = -1
        frag = "block_tables[1][0] = -1 "
    elif kind == "len_past_table":
        sl[0] = bt.shape[1] * BS + 1
        frag = f"seq_lens[0] = {int(sl[0])} "
    elif kind == "mt_last_block":
        j = (nb[last] - 1) // BS
        mt[last, j] = nmeta
        frag = f"metadata_block_tables[{last}][{j}] = {nmeta} "
    elif kind == "mt_past_length":
        b = next(b for b in range(wl.B) if -(-nb[b] // BS) < mt.shape[1])
        mt[b, -(-nb[b] // BS)] = -3
    else:
        raise ValueError(kind)
    return bt, sl, mt, frag


KINDS = ["valid", "bt_last_block", "bt_negative", "bt_past_length", "two_requests", "len_past_table",
         "mt_last_block", "mt_past_length"]


def oracle_verdict(fn):
    try:
        fn()
        return True
    except ValueError:
        return False


def checked_verdict(qs, fn):
    with qs.checked_calls():
        try:
            fn()
            torch.cuda.synchronize()
            return True, ""
        except qs.QsError as e:
            assert e.status == qs.QS_ERR_INVALID, str(e)
            return False, str(e)


def judge(qs, name, kind, frag, o_ok, run_checked, run_plain, outputs, exact=True, frag_applies=True):
    """run_checked / run_plain fill `outputs()` (fresh sentinel tensors each time) and return them."""
    say(f"checked build: {name} / {kind}")
    outs_c = []
    c_ok, msg = checked_verdict(qs, lambda: outs_c.append(run_checked()))
    if exact:
        assert c_ok == o_ok, f"{name}/{kind}: checked {c_ok}, oracle {o_ok}: {msg}"
    else:
        assert o_ok or not c_ok, f"{name}/{kind}: oracle refuses, checked build accepts"
    if not c_ok:
        assert msg.split("] ", 1)[1].startswith(name), msg
        if frag is not None and frag_applies:
            assert frag in msg, (frag, msg)
        untouched = outputs()
        for t in untouched:
            assert torch.equal(t, outputs.fresh(t)), f"{name}/{kind}: a refused call wrote its output"
    else:
        got = outs_c[0]
        ref = run_plain()
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"{name}/{kind}: checked and plain builds differ"


class Outs:
    """Sentinel-filled outputs of one call; `fresh(t)` is what an untouched one holds."""

    def __init__(self, *specs):
        self.specs = specs
        self.last = None

    def __call__(self):
        return self.last

    def make(self):
        self.last = [torch.full(shape, SENT if dt.is_floating_point else -5, dtype=dt, device=DEV)
                     for shape, dt in self.specs]
        return self.last

    def fresh(self, t):
        return torch.full_like(t, SENT if t.dtype.is_floating_point else -5)


def base_case(dtype=torch.float32):
    # three requests, one long enough to span five metadata blocks; spare table slots in every row
    return W.random_case(91, 3, 16, 4, 16, [16 * 40 + 5, 16 * 9, 16 * 68 + 3], k=8, dtype=dtype,
                         with_importance=True, spare_blocks=5)


def widen_tables(wl, extra=3):
    """Two more block-table and metadata-table columns (zeros), so 'past length' slots exist in every row."""
    z = torch.zeros((wl.B, extra), dtype=torch.int32)
    wl.block_tables = torch.cat([wl.block_tables, z], 1)
    wl.meta_tables = torch.cat([wl.meta_tables, z[:, :1]], 1)
    return wl


@pytest.fixture(scope="module")
def case():
    wl = widen_tables(base_case())
    wl.meta_seq_lens = wl.seq_lens.clone()
    return wl


# ------------------------------------------------------------------------------------------
# one test per call
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("kind", KINDS)
def test_checked_build_metadata(qs, oracle, case, kind):
    wl = case
    bt, sl, mt, frag = mutate(kind, wl)
    shape = (wl.num_meta_blocks, wl.BS, wl.N, wl.D)
    s = torch.full(shape, SENT)
    o_ok = oracle_verdict(lambda: oracle.build_metadata(wl.k_cache, bt, sl, mt, wl.num_meta_blocks, maxb=s, minb=s))
    outs = Outs((shape, torch.float32), (shape, torch.float32))
    kc, btd, sld, mtd = wl.k_cache.to(DEV), bt.to(DEV), sl.to(DEV), mt.to(DEV)

    def run():
        mx, mn = outs.make()
        qs.qs_build_metadata(kc, btd, sld, mtd, mx, mn)
        return mx, mn
    judge(qs, "qs_build_metadata", kind, frag, o_ok, run, run, outs)


@pytest.mark.parametrize("kind", KINDS)
def test_checked_update_metadata(qs, oracle, case, kind):
    wl = case
    bt, sl, mt, frag = mutate(kind, wl)
    nb = nbs(sl, wl.BS)
    # refresh the last two blocks of every request: planted entries there are used, others not
    fb = torch.tensor([max(n - 2, 0) for n in nb], dtype=torch.int32)
    shape = (wl.num_meta_blocks, wl.BS, wl.N, wl.D)
    s = torch.full(shape, SENT)
    o_ok = oracle_verdict(lambda: oracle.update_metadata(wl.k_cache, bt, sl, fb, 2, mt, s.clone(), s.clone()))
    outs = Outs((shape, torch.float32), (shape, torch.float32))
    kc, btd, sld, mtd, fbd = wl.k_cache.to(DEV), bt.to(DEV), sl.to(DEV), mt.to(DEV), fb.to(DEV)

    def run():
        mx, mn = outs.make()
        qs.qs_update_metadata(kc, btd, sld, fbd, 2, mtd, mx, mn)
        return mx, mn
    judge(qs, "qs_update_metadata", kind, frag, o_ok, run, run, outs, frag_applies=kind != "two_requests")


def built_metadata(qs, wl):
    shape = (wl.num_meta_blocks, wl.BS, wl.N, wl.D)
    mx = torch.zeros(shape, device=DEV)
    mn = torch.zeros(shape, device=DEV)
    qs.qs_build_metadata(wl.k_cache.to(DEV), wl.block_tables.to(DEV), wl.seq_lens.to(DEV), wl.meta_tables.to(DEV),
                         mx, mn)
    return mx, mn


@pytest.mark.parametrize("flags", [0, 3])
@pytest.mark.parametrize("kind", KINDS)
def test_checked_block_select(qs, oracle, case, kind, flags):
    wl = case
    bt, sl, mt, frag = mutate(kind, wl)
    mx, mn = built_metadata(qs, wl)
    ts = torch.tensor([5, 40, 0], dtype=torch.int32)
    k = wl.k
    o_ok = oracle_verdict(lambda: oracle.block_select(wl.query, mx.cpu(), mn.cpu(), mt, sl, k, tsmu=ts, flags=flags))
    outs = Outs(((wl.B, wl.N, k), torch.int32), ((wl.B, wl.N), torch.int32))
    q, mtd, sld, tsd = wl.query.to(DEV), mt.to(DEV), sl.to(DEV), ts.to(DEV)

    def run():
        sel, ns = outs.make()
        qs.qs_block_select(q, mx, mn, mtd, sld, k, tokens_since_update=tsd, flags=flags, selected=sel, n_selected=ns)
        return sel, ns
    # the select reads no block_tables: only metadata-table and length plants can be refused
    judge(qs, "qs_block_select", kind, frag, o_ok, run, run, outs, exact=flags == 0,
          frag_applies=kind.startswith("mt"))


@pytest.mark.parametrize("kind", KINDS)
def test_checked_probe_select(qs, oracle, case, kind):
    wl = case
    bt, sl, mt, frag = mutate(kind, wl)
    k = 6
    o_ok = oracle_verdict(lambda: oracle.probe_select(wl.query, wl.k_cache, bt, sl, k, wl.N,
                                                      importance=wl.importance, n_probe=8, flags=oracle.RECENCY))
    outs = Outs(((wl.B, wl.H, k), torch.int32), ((wl.B, wl.H), torch.int32))
    q, kc, btd, sld, imp = wl.query.to(DEV), wl.k_cache.to(DEV), bt.to(DEV), sl.to(DEV), wl.importance.to(DEV)

    def run():
        sel, ns = outs.make()
        qs.qs_probe_select(q, kc, btd, sld, k, importance=imp, n_probe=8, flags=qs.QS_RECENCY, selected=sel,
                           n_selected=ns)
        return sel, ns
    judge(qs, "qs_probe_select", kind, frag, o_ok, run, run, outs, frag_applies=not kind.startswith("mt"))


ATTN_KINDS = ["valid", "bt_selected", "bt_not_selected", "bt_selected_past_count", "len_past_table"]


@pytest.mark.parametrize("kind", ATTN_KINDS)
def test_checked_sparse_attn(qs, oracle, case, kind):
    wl = case
    bt, sl = wl.block_tables.clone(), wl.seq_lens.clone()
    nkv = wl.k_cache.shape[0]
    k = 5
    # selection: rows of each request pick blocks 0, 2, 4, ... (ascending), row 1 of each request one fewer
    nb = nbs(sl, wl.BS)
    sel = torch.full((wl.B, wl.N, k), -1, dtype=torch.int32)
    ns = torch.zeros((wl.B, wl.N), dtype=torch.int32)
    for b in range(wl.B):
        picks = list(range(0, nb[b], 2))[:k]
        for r in range(wl.N):
            m = len(picks) - (1 if r == 1 and picks else 0)
            sel[b, r, :len(picks)] = torch.tensor(picks, dtype=torch.int32)
            ns[b, r] = m
    frag = None
    if kind == "bt_selected":
        blk = int(sel[2, 0, 1])
        bt[2, blk] = nkv + 1
        frag = f"block_tables[2][{blk}] = {nkv + 1} "
    elif kind == "bt_not_selected":
        bt[2, 1] = -1                       # odd blocks are never selected
    elif kind == "bt_selected_past_count":
        # the last slot of row 1 is below k but past its n_selected; every other row selects it
        nrow = int(ns[1, 1])
        blk = int(sel[1, 1, nrow])
        for r in range(wl.N):
            if r != 1:
                sel[1, r, nrow] = -1
                ns[1, r] = nrow
        bt[1, blk] = nkv
    elif kind == "len_past_table":
        sl[0] = bt.shape[1] * wl.BS + 1      # attention reads no length rule: accepted
    o_ok = oracle_verdict(lambda: oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, bt, sl, sel, ns, wl.N))
    outs = Outs(((wl.B, wl.H, wl.D), torch.float32))
    q, kc, vc, btd, sld, seld, nsd = (t.to(DEV) for t in (wl.query, wl.k_cache, wl.v_cache, bt, sl, sel, ns))

    def run():
        (out,) = outs.make()
        qs.qs_sparse_attn_decode(q, kc, vc, btd, sld, seld, nsd, out=out)
        return (out,)
    judge(qs, "qs_sparse_attn_decode", kind, frag, o_ok, run, run, outs)


@pytest.mark.parametrize("kind", KINDS)
def test_checked_select_attn(qs, oracle, case, kind):
    wl = case
    bt, sl, mt, frag = mutate(kind, wl)
    mx, mn = built_metadata(qs, wl)
    k = wl.k

    def oracle_call():
        osel, ons, _ = oracle.block_select(wl.query, mx.cpu(), mn.cpu(), mt, sl, k)
        oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, bt, sl, osel, ons, wl.N)
    o_ok = oracle_verdict(oracle_call)
    outs = Outs(((wl.B, wl.H, wl.D), torch.float32), ((wl.B, wl.N, k), torch.int32), ((wl.B, wl.N), torch.int32))
    q, kc, vc, btd, sld, mtd = (t.to(DEV) for t in (wl.query, wl.k_cache, wl.v_cache, bt, sl, mt))

    def run():
        out, sel, ns = outs.make()
        qs.qs_select_attn_decode(q, mx, mn, mtd, kc, vc, btd, sld, k, out=out, selected=sel, n_selected=ns)
        return out, sel, ns
    judge(qs, "qs_select_attn_decode", kind, frag, o_ok, run, run, outs, exact=False)


@pytest.mark.parametrize("kind", KINDS)
def test_checked_probe_attn(qs, oracle, case, kind):
    wl = case
    bt, sl, mt, frag = mutate(kind, wl)
    k = 6

    def oracle_call():
        o = oracle.probe_select(wl.query, wl.k_cache, bt, sl, k, wl.N, importance=wl.importance, n_probe=8,
                                flags=oracle.RECENCY)
        oracle.sparse_attn_decode(wl.query, wl.k_cache, wl.v_cache, bt, sl, o["selected"], o["n_selected"], wl.H)
    o_ok = oracle_verdict(oracle_call)
    outs = Outs(((wl.B, wl.H, wl.D), torch.float32), ((wl.B, wl.H, k), torch.int32), ((wl.B, wl.H), torch.int32))
    q, kc, vc, btd, sld, imp = (t.to(DEV) for t in (wl.query, wl.k_cache, wl.v_cache, bt, sl, wl.importance))

    def run():
        out, sel, ns = outs.make()
        qs.qs_probe_attn_decode(q, kc, vc, btd, sld, k, importance=imp, n_probe=8, flags=qs.QS_RECENCY, out=out,
                                selected=sel, n_selected=ns)
        return out, sel, ns
    judge(qs, "qs_probe_attn_decode", kind, frag, o_ok, run, run, outs, frag_applies=not kind.startswith("mt"))


@pytest.mark.parametrize("kind", ["valid", "bt_last_block", "bt_negative", "bt_past_length", "two_requests",
                                  "len_past_table"])
def test_checked_prefill_importance(qs, oracle, kind):
    wl = widen_tables(W.random_case(92, 3, 4, 2, 16, [16 * 5 + 3, 16 * 2, 16 * 6], k=2, with_v=False))
    bt, sl, mt, frag = mutate(kind, wl)
    q = W.prefill_queries(wl, 92)
    stride = q.shape[1]
    o_ok = oracle_verdict(lambda: oracle.prefill_importance(q, wl.k_cache, bt, sl, wl.N, stride=stride))
    outs = Outs(((wl.B, stride), torch.float32))
    qd, kc, btd, sld = (t.to(DEV) for t in (q, wl.k_cache, bt, sl))

    def run():
        (imp,) = outs.make()
        qs.qs_prefill_importance(qd, kc, btd, sld, importance=imp, importance_stride=stride)
        return (imp,)
    judge(qs, "qs_prefill_importance", kind, frag, o_ok, run, run, outs)


def test_checked_build_refuses_capture(qs, case):
    """Under stream capture the checked build refuses (it must wait for its check) and leaves the capture intact."""
    wl = case
    mx, mn = built_metadata(qs, wl)
    q, mtd, sld = wl.query.to(DEV), wl.meta_tables.to(DEV), wl.seq_lens.to(DEV)
    sel = torch.empty((wl.B, wl.N, wl.k), dtype=torch.int32, device=DEV)
    ns = torch.empty((wl.B, wl.N), dtype=torch.int32, device=DEV)
    qs.qs_block_select(q, mx, mn, mtd, sld, wl.k, selected=sel, n_selected=ns)   # workspace sized before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    status = None
    with torch.cuda.stream(s):
        g.capture_begin()
        try:
            with qs.checked_calls():
                try:
                    qs.qs_block_select(q, mx, mn, mtd, sld, wl.k, selected=sel, n_selected=ns)
                except qs.QsError as e:
                    status = e.status
        finally:
            g.capture_end()
    torch.cuda.synchronize()
    assert status == qs.QS_ERR_UNSUPPORTED
