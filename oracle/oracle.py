"""ctypes front end of the C oracle (``qs_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path. It takes numpy arrays / CPU torch tensors
(bf16 is passed as its raw 16-bit patterns), calls the plain C loops and returns numpy
results. It imports nothing from the HIP package.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qs_oracle.c")
LIB = os.path.join(HERE, "libqsoracle.so")

F32, BF16, I8, F16 = 0, 1, 2, 3
FORCE_SINK, FORCE_WINDOW, RECENCY = 1, 2, 4


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.qso_build_metadata.argtypes = [i, i, i, i, i, P, i, P, i, P, P, i, P, P, i]
        L.qso_update_metadata.argtypes = [i, i, i, i, i, P, i, P, i, P, P, i, P, i, P, P, i]
        L.qso_block_select.argtypes = [i, i, i, i, i, i, P, P, P, P, i, i, P, P, ctypes.c_uint, i, P, P, P]
        L.qso_probe_select.argtypes = [i, i, i, i, i, i, i, P, P, i, P, i, P, P, i, i, i, ctypes.c_uint,
                                       P, P, P, P, P, P]
        L.qso_sparse_attn_decode.argtypes = [i, i, i, i, i, i, i, P, P, P, P, P, i, P, i, P, P, P, i, i,
                                             ctypes.c_double, P]
        L.qso_quantize_row_i8.argtypes = [P, i, P, P]
        L.qso_widen.argtypes = [i, P, i, P]
        L.qso_prefill_importance.argtypes = [i, i, i, i, i, i, P, i, P, i, P, i, P, ctypes.c_double, i, i, P, P, i]
        L.qso_prefill_importance.restype = ctypes.c_int
        L.qso_widen.restype = None
        for f in (L.qso_build_metadata, L.qso_block_select, L.qso_probe_select, L.qso_sparse_attn_decode):
            f.restype = ctypes.c_int
        L.qso_quantize_row_i8.restype = None
        _lib = L
    return _lib


# ------------------------------------------------------------------------------------------
# marshalling helpers
# ------------------------------------------------------------------------------------------

def _np(x):
    """numpy view of a CPU torch tensor or a numpy array; bf16 becomes uint16 bits."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16)
            return x.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x)


def _dtype_code(a) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.int8:
        return I8
    if a.dtype == np.float16:
        return F16
    raise TypeError(f"unsupported dtype {a.dtype}")


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    return None if a is None else np.ascontiguousarray(_np(a), dtype=np.int32)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid input (rc={rc})")


# ------------------------------------------------------------------------------------------
# the four operations
# ------------------------------------------------------------------------------------------

def build_metadata(k_cache, block_tables, seq_lens, meta_tables, num_meta_blocks,
                   maxb=None, minb=None):
    """O1. Returns (maxb, minb) [num_meta_blocks, BS, N, D] in k_cache's dtype (numpy;
    bf16 as uint16 bits). ``maxb``/``minb`` may be given as initial contents (rows the
    method does not write keep them)."""
    kc = np.ascontiguousarray(_np(k_cache))
    nkv, BS, N, D = kc.shape
    bt, sl, mt = _i32(block_tables), _i32(seq_lens), _i32(meta_tables)
    B = sl.shape[0]
    shape = (num_meta_blocks, BS, N, D)
    mx = np.zeros(shape, kc.dtype) if maxb is None else np.array(_np(maxb), dtype=kc.dtype, copy=True)
    mn = np.zeros(shape, kc.dtype) if minb is None else np.array(_np(minb), dtype=kc.dtype, copy=True)
    rc = lib().qso_build_metadata(B, N, D, BS, _dtype_code(kc), _p(kc), nkv, _p(bt), bt.shape[1],
                                  _p(sl), _p(mt), mt.shape[1], _p(mx), _p(mn), num_meta_blocks)
    _check(rc, "build_metadata")
    return mx, mn


def update_metadata(k_cache, block_tables, seq_lens, first_block, max_new_blocks, meta_tables, maxb, minb):
    """O1' (refresh). Returns copies of (maxb, minb) with sequence blocks first_block[b] ..
    min(nb, first_block[b] + max_new_blocks) - 1 of each request recomputed."""
    kc = np.ascontiguousarray(_np(k_cache))
    nkv, BS, N, D = kc.shape
    bt, sl, mt, fb = _i32(block_tables), _i32(seq_lens), _i32(meta_tables), _i32(first_block)
    B = sl.shape[0]
    mx = np.array(_np(maxb), dtype=kc.dtype, copy=True)
    mn = np.array(_np(minb), dtype=kc.dtype, copy=True)
    rc = lib().qso_update_metadata(B, N, D, BS, _dtype_code(kc), _p(kc), nkv, _p(bt), bt.shape[1], _p(sl),
                                   _p(fb), int(max_new_blocks), _p(mt), mt.shape[1], _p(mx), _p(mn), mx.shape[0])
    _check(rc, "update_metadata")
    return mx, mn


def block_select(query, maxb, minb, meta_tables, seq_lens, k, H=None, tsmu=None, flags=0):
    """O2. Returns (selected [B,N,k] int32, n_selected [B,N] int32, scores [B,N,MMBPR*BS] f64)."""
    q = np.ascontiguousarray(_np(query))
    mx, mn = np.ascontiguousarray(_np(maxb)), np.ascontiguousarray(_np(minb))
    assert q.dtype == mx.dtype == mn.dtype
    B, Hq, D = q.shape
    nmeta, BS, N, D2 = mx.shape
    assert D == D2
    mt, sl, ts = _i32(meta_tables), _i32(seq_lens), _i32(tsmu)
    mmbpr = mt.shape[1]
    sel = np.empty((B, N, k), np.int32)
    nsel = np.empty((B, N), np.int32)
    sc = np.empty((B, N, mmbpr * BS), np.float64)
    rc = lib().qso_block_select(B, Hq, N, D, BS, _dtype_code(q), _p(q), _p(mx), _p(mn), _p(mt), mmbpr,
                                nmeta, _p(sl), _p(ts), flags, k, _p(sel), _p(nsel), _p(sc))
    _check(rc, "block_select")
    return sel, nsel, sc


def probe_select(query, k_cache, block_tables, seq_lens, k, N, importance=None, n_probe=8,
                 flags=RECENCY):
    """O3. Returns dict(selected [B,H,k], n_selected [B,H], probe [B,H,MKBPR] f64,
    imp_sum [B,MKBPR] f32, n_imp [B,H], kind [B,H,MKBPR] int8 (0 none, 1 importance,
    2 probe, 3 recency-added, 4 evicted by recency))."""
    q = np.ascontiguousarray(_np(query))
    kc = np.ascontiguousarray(_np(k_cache))
    B, H, D = q.shape
    nkv, BS, N2, D2 = kc.shape
    assert N2 == N and D2 == D
    bt, sl = _i32(block_tables), _i32(seq_lens)
    mkbpr = bt.shape[1]
    imp = None if importance is None else np.ascontiguousarray(_np(importance), dtype=np.float32)
    stride = 0 if imp is None else imp.shape[1]
    sel = np.empty((B, H, k), np.int32)
    nsel = np.empty((B, H), np.int32)
    probe = np.empty((B, H, mkbpr), np.float64)
    imps = np.zeros((B, mkbpr), np.float32)
    nimp = np.empty((B, H), np.int32)
    kind = np.zeros((B, H, mkbpr), np.int8)
    rc = lib().qso_probe_select(B, H, N, D, BS, _dtype_code(q), _dtype_code(kc), _p(q), _p(kc), nkv,
                                _p(bt), mkbpr, _p(sl), _p(imp), stride, n_probe, k, flags,
                                _p(sel), _p(nsel), _p(probe), _p(imps), _p(nimp), _p(kind))
    _check(rc, "probe_select")
    return dict(selected=sel, n_selected=nsel, probe=probe, imp_sum=imps, n_imp=nimp, kind=kind)


def sparse_attn_decode(query, k_cache, v_cache, block_tables, seq_lens, selected, n_selected,
                       sel_heads, softmax_scale=0.0, k_scale=None, v_scale=None):
    """O4. Returns out [B, H, D] float64."""
    q = np.ascontiguousarray(_np(query))
    kc, vc = np.ascontiguousarray(_np(k_cache)), np.ascontiguousarray(_np(v_cache))
    assert kc.dtype == vc.dtype
    B, H, D = q.shape
    nkv, BS, N, D2 = kc.shape
    bt, sl = _i32(block_tables), _i32(seq_lens)
    sel, nsel = _i32(selected), _i32(n_selected)
    k = sel.shape[-1]
    ks = None if k_scale is None else np.ascontiguousarray(_np(k_scale), dtype=np.float32)
    vs = None if v_scale is None else np.ascontiguousarray(_np(v_scale), dtype=np.float32)
    out = np.empty((B, H, D), np.float64)
    rc = lib().qso_sparse_attn_decode(B, H, N, D, BS, _dtype_code(q), _dtype_code(kc), _p(q), _p(kc),
                                      _p(vc), _p(ks), _p(vs), nkv, _p(bt), bt.shape[1], _p(sl),
                                      _p(sel), _p(nsel), sel_heads, k, float(softmax_scale), _p(out))
    _check(rc, "sparse_attn_decode")
    return out


def prefill_importance(query, k_cache, block_tables, seq_lens, N, softmax_scale=0.0, heads=None, stride=None):
    """O5. query [B, max_len, H, D]. Returns (importance [B, stride] f64, head_imp [B, H, stride] f64);
    ``heads`` = (lo, hi) restricts the computation to heads lo .. hi-1 (importance then sums those)."""
    q = np.ascontiguousarray(_np(query))
    kc = np.ascontiguousarray(_np(k_cache))
    assert q.dtype == kc.dtype
    B, max_len, H, D = q.shape
    nkv, BS, N2, D2 = kc.shape
    assert N2 == N and D2 == D
    bt, sl = _i32(block_tables), _i32(seq_lens)
    stride = max_len if stride is None else stride
    lo, hi = (0, H) if heads is None else heads
    imp = np.zeros((B, stride), np.float64)
    himp = np.zeros((B, H, stride), np.float64)
    rc = lib().qso_prefill_importance(B, H, N, D, BS, _dtype_code(q), _p(q), max_len, _p(kc), nkv, _p(bt),
                                      bt.shape[1], _p(sl), float(softmax_scale), lo, hi, _p(imp), _p(himp), stride)
    _check(rc, "prefill_importance")
    return imp, himp


def widen(a):
    """The oracle's exact widening of stored elements (f32, bf16 bits, f16, int8) to float64."""
    a = np.ascontiguousarray(_np(a))
    out = np.empty(a.size, np.float64)
    lib().qso_widen(_dtype_code(a), _p(a), a.size, _p(out))
    return out.reshape(a.shape)


def quantize_row_i8(x):
    """The oracle's int8 query quantiser on one fp32 row: (codes int8, scale float)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(x.shape[0], np.int8)
    s = np.zeros(1, np.float32)
    lib().qso_quantize_row_i8(_p(x), x.shape[0], _p(codes), _p(s))
    return codes, float(s[0])
