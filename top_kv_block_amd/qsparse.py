"""Python binding of libqsparse.so (the C ABI in include/qsparse.h).

Argument marshalling only: shape/dtype/device checks on torch tensors, output and
workspace allocation, and the call on torch's current HIP stream. Every step of the
computation runs in the library's HIP kernels; there is no fallback. Importing this
module fails loudly if the library has not been built (python -m top_kv_block_amd.build).

QSPARSE_CHECKED=1 in the environment loads the checked build instead, whose calls first
check the device-resident tables they will use (and wait for that check);
`checked_calls()` switches to it for a block of code.
"""

from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqsparse.so")
_LIB_CHECKED_PATH = os.path.join(_HERE, "libqsparse_checked.so")

QS_OK, QS_ERR_INVALID, QS_ERR_UNSUPPORTED, QS_ERR_HIP = 0, 1, 2, 3
QS_F32, QS_BF16, QS_I8, QS_F16 = 0, 1, 2, 3
QS_FORCE_SINK, QS_FORCE_WINDOW, QS_RECENCY = 1, 2, 4

# the C ABI's exported functions (also checked by the ABI tests)
EXPORTS = (
    "qs_build_metadata", "qs_update_metadata", "qs_block_select_workspace_bytes", "qs_block_select",
    "qs_probe_select_workspace_bytes", "qs_probe_select",
    "qs_sparse_attn_workspace_bytes", "qs_sparse_attn_decode", "qs_select_attn_workspace_bytes",
    "qs_select_attn_decode", "qs_select_attn_decode_static", "qs_probe_attn_workspace_bytes", "qs_probe_attn_decode",
    "qs_prefill_importance_workspace_bytes", "qs_prefill_importance", "qs_last_error", "qs_version",
    "qs_checked_build",
)


class QsError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


def _load(path):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m top_kv_block_amd.build` "
                          "(the HIP path has no fallback)")
    lib = ctypes.CDLL(path)
    P, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    lib.qs_build_metadata.argtypes = [i32, i32, i32, i32, ctypes.c_int, P, i32, P, i32, P, P, i32, P, P, i32, P]
    lib.qs_update_metadata.argtypes = [i32, i32, i32, i32, ctypes.c_int, P, i32, P, i32, P, P, i32, P, i32, P, P,
                                       i32, P]
    lib.qs_block_select_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.qs_block_select_workspace_bytes.restype = sz
    lib.qs_block_select.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, P, P, P, i32, P, i32, P, P, u32, i32,
                                    P, P, P, P, sz, P]
    lib.qs_probe_select.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, P, P, i32, P, i32, P, P,
                                    i32, i32, i32, u32, P, P, P, P, sz, P]
    lib.qs_probe_select_workspace_bytes.argtypes = [i32, i32, i32]
    lib.qs_probe_select_workspace_bytes.restype = sz
    lib.qs_sparse_attn_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.qs_sparse_attn_workspace_bytes.restype = sz
    lib.qs_sparse_attn_decode.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, P, P, P, P, P, i32,
                                          P, i32, P, P, P, i32, i32, ctypes.c_float, P, P, sz, P]
    lib.qs_select_attn_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.c_int]
    lib.qs_select_attn_workspace_bytes.restype = sz
    lib.qs_select_attn_decode.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, P, P, P, i32, P, i32, P, P, i32, P,
                                          i32, P, P, u32, i32, ctypes.c_float, P, P, P, P, sz, P]
    lib.qs_select_attn_decode_static.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, P, P, P, i32, P, i32, P, P,
                                                 i32, P, i32, P, P, u32, i32, ctypes.c_float, P, P, P, P]
    lib.qs_probe_attn_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.qs_probe_attn_workspace_bytes.restype = sz
    lib.qs_probe_attn_decode.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, P, P, P, P, P, P,
                                         ctypes.c_int, i32, P, i32, P, P, i32, i32, i32, u32, ctypes.c_float, P, P, P,
                                         P, sz, P]
    lib.qs_prefill_importance_workspace_bytes.argtypes = [i32, i32, i32]
    lib.qs_prefill_importance_workspace_bytes.restype = sz
    lib.qs_prefill_importance.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, P, i32, P, i32, P, i32, P,
                                          ctypes.c_float, P, i32, P, P, sz, P]
    for f in ("qs_build_metadata", "qs_update_metadata", "qs_block_select", "qs_probe_select",
              "qs_sparse_attn_decode", "qs_select_attn_decode", "qs_select_attn_decode_static", "qs_probe_attn_decode",
              "qs_prefill_importance"):
        getattr(lib, f).restype = ctypes.c_int
    lib.qs_last_error.restype = ctypes.c_char_p
    lib.qs_version.restype = ctypes.c_char_p
    lib.qs_checked_build.restype = ctypes.c_int32
    return lib


lib = _load(_LIB_CHECKED_PATH if os.environ.get("QSPARSE_CHECKED", "0") not in ("", "0") else _LIB_PATH)
_checked_lib = None


def load_checked():
    """The checked build (loaded on first use)."""
    global _checked_lib
    if _checked_lib is None:
        _checked_lib = _load(_LIB_CHECKED_PATH)
    return _checked_lib


@contextlib.contextmanager
def checked_calls():
    """Routes this module's calls through the checked build inside the block (not thread-safe)."""
    global lib
    saved, lib = lib, load_checked()
    try:
        yield lib
    finally:
        lib = saved


def _check(status):
    if status != QS_OK:
        raise QsError(status, lib.qs_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()  # the argtypes convert it to void*


def _dtype_code(t):
    if t.dtype == torch.float32:
        return QS_F32
    if t.dtype == torch.bfloat16:
        return QS_BF16
    if t.dtype == torch.int8:
        return QS_I8
    if t.dtype == torch.float16:
        return QS_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
    return dev


def _i32(t, name):
    if t is not None and t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _rows(t, B, name, width=None):
    """t must be a [>=B, width] (or [>=B]) table."""
    if t is None:
        return
    _need(t.dim() >= 1 and t.shape[0] >= B, f"{name} needs at least {B} rows")
    if width is not None:
        _need(t.dim() == 2 and t.shape[1] == width, f"{name} must have {width} columns")


# torch's current stream as a raw handle: the private accessor returns the pointer
# without building a Stream object (a few microseconds a call); the public API otherwise
_raw_stream_of = getattr(torch._C, "_cuda_getCurrentRawStream", None)
if _raw_stream_of is None:
    def _raw_stream_of(index):
        return torch.cuda.current_stream(index).cuda_stream


def _index(dev):
    dev = torch.device(dev)
    return dev.index if dev.index is not None else torch.cuda.current_device()


def _stream(dev):
    return _raw_stream_of(_index(dev))


_ws_sizes = {}


def _ws_bytes(fn, *args):
    """A workspace-size query of the loaded library, remembered per argument tuple."""
    key = (id(lib), fn, args)
    n = _ws_sizes.get(key)
    if n is None:
        n = _ws_sizes[key] = getattr(lib, fn)(*args)
    return n


_workspaces = {}
_retired = []


def workspace(nbytes, device, op, stream=None):
    """An uninitialised, 256-byte aligned workspace cached per (device, stream, operation)
    and grown on demand, so that calls of one operation on different streams never share
    scratch memory (calls on one stream are ordered). A workspace that is replaced by a
    larger one stays allocated: a HIP graph captured with it keeps a valid address. It
    grows at least twofold each time, so what stays allocated is under twice the largest
    workspace of each (device, stream, operation).

    Under stream capture every call gets a workspace of its own instead, allocated from the
    graph's private memory pool, which the graph keeps until it is destroyed: graphs
    captured on one stream (torch captures on a shared side stream by default) then never
    share scratch memory, so they may be replayed concurrently on different streams.
    ``stream``: the raw handle of the current stream, when the caller has it already."""
    dev = torch.device(device)
    index = dev.index if dev.index is not None else torch.cuda.current_device()
    if torch.cuda.is_current_stream_capturing():
        return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)
    key = (index, _raw_stream_of(index) if stream is None else stream, op)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        size = max(int(nbytes), 256)
        if ws is not None:
            _retired.append(ws)
            size = max(size, 2 * ws.numel())
        ws = torch.empty(size, dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


# ------------------------------------------------------------------------------------------
# the operations (names and argument meaning as in include/qsparse.h)
# ------------------------------------------------------------------------------------------

def _meta_shapes(k_cache, block_tables, seq_lens, metadata_block_tables, maxblocks, minblocks):
    for n, t in (("block_tables", block_tables), ("seq_lens", seq_lens),
                 ("metadata_block_tables", metadata_block_tables)):
        _i32(t, n)
    if maxblocks.shape != minblocks.shape or maxblocks.shape[1:] != k_cache.shape[1:]:
        raise ValueError("maxblocks/minblocks must be [num_meta_blocks, BS, N, D]")
    if maxblocks.dtype != k_cache.dtype or minblocks.dtype != k_cache.dtype:
        raise TypeError("metadata dtype must match k_cache")
    B = seq_lens.shape[0]
    _rows(block_tables, B, "block_tables")
    _rows(metadata_block_tables, B, "metadata_block_tables")
    return B


def qs_build_metadata(k_cache, block_tables, seq_lens, metadata_block_tables, maxblocks, minblocks):
    """Per-block, per-channel max/min of K into the paged metadata blocks (in place)."""
    dev = _dev(k_cache, block_tables, seq_lens, metadata_block_tables, maxblocks, minblocks)
    B = _meta_shapes(k_cache, block_tables, seq_lens, metadata_block_tables, maxblocks, minblocks)
    nkv, BS, N, D = k_cache.shape
    _check(lib.qs_build_metadata(B, N, D, BS, _dtype_code(k_cache), _ptr(k_cache), nkv, _ptr(block_tables),
                                 block_tables.shape[1], _ptr(seq_lens), _ptr(metadata_block_tables),
                                 metadata_block_tables.shape[1], _ptr(maxblocks), _ptr(minblocks),
                                 maxblocks.shape[0], _stream(dev)))


def qs_update_metadata(k_cache, block_tables, seq_lens, first_block, max_new_blocks, metadata_block_tables,
                       maxblocks, minblocks):
    """Recompute the metadata of blocks first_block[b] .. first_block[b] + max_new_blocks - 1
    (those below ceil(seq_lens[b] / BS)) of each request, in place; nothing else is written."""
    dev = _dev(k_cache, block_tables, seq_lens, first_block, metadata_block_tables, maxblocks, minblocks)
    B = _meta_shapes(k_cache, block_tables, seq_lens, metadata_block_tables, maxblocks, minblocks)
    _i32(first_block, "first_block")
    _rows(first_block, B, "first_block")
    nkv, BS, N, D = k_cache.shape
    _check(lib.qs_update_metadata(B, N, D, BS, _dtype_code(k_cache), _ptr(k_cache), nkv, _ptr(block_tables),
                                  block_tables.shape[1], _ptr(seq_lens), _ptr(first_block), int(max_new_blocks),
                                  _ptr(metadata_block_tables), metadata_block_tables.shape[1], _ptr(maxblocks),
                                  _ptr(minblocks), maxblocks.shape[0], _stream(dev)))


def block_select_workspace_bytes(B, N, block_size, mmbpr):
    return _ws_bytes("qs_block_select_workspace_bytes", B, N, block_size, mmbpr)


def qs_block_select(query, maxblocks, minblocks, metadata_block_tables, seq_lens, k,
                    tokens_since_update=None, flags=0, selected=None, n_selected=None,
                    block_scores=None, workspace_buf=None):
    """Quest top-k selection. Returns (selected [B, N, k] int32, n_selected [B, N] int32)."""
    dev = _dev(query, maxblocks, minblocks, metadata_block_tables, seq_lens, tokens_since_update,
               selected, n_selected, block_scores)
    for n, t in (("metadata_block_tables", metadata_block_tables), ("seq_lens", seq_lens),
                 ("tokens_since_update", tokens_since_update)):
        _i32(t, n)
    B, H, D = query.shape
    nmeta, BS, N, D2 = maxblocks.shape
    mmbpr = metadata_block_tables.shape[1]
    _need(D2 == D and H % N == 0, "query and metadata shapes disagree")
    _need(maxblocks.shape == minblocks.shape and maxblocks.dtype == minblocks.dtype == query.dtype,
          "maxblocks/minblocks must match each other and the query dtype")
    _rows(metadata_block_tables, B, "metadata_block_tables")
    _rows(seq_lens, B, "seq_lens")
    _rows(tokens_since_update, B, "tokens_since_update")
    if selected is None:
        selected = torch.empty((B, N, k), dtype=torch.int32, device=dev)
    if n_selected is None:
        n_selected = torch.empty((B, N), dtype=torch.int32, device=dev)
    _need(selected.numel() >= B * N * k and n_selected.numel() >= B * N, "selected must hold [B, N, k]")
    if block_scores is not None and (block_scores.dtype != torch.float32 or
                                     block_scores.numel() < B * N * mmbpr * BS):
        raise ValueError("block_scores must be fp32 [B, N, MMBPR*BS]")
    nbytes = block_select_workspace_bytes(B, N, BS, mmbpr)
    st = _stream(dev)
    ws = workspace_buf if workspace_buf is not None else workspace(nbytes, dev, "select", st)
    _check(lib.qs_block_select(B, H, N, D, BS, _dtype_code(query), _ptr(query), _ptr(maxblocks),
                               _ptr(minblocks), nmeta, _ptr(metadata_block_tables), mmbpr, _ptr(seq_lens),
                               _ptr(tokens_since_update), int(flags), int(k), _ptr(selected), _ptr(n_selected),
                               _ptr(block_scores), _ptr(ws), ws.numel(), st))
    return selected, n_selected


def probe_select_workspace_bytes(B, H, mkbpr):
    return _ws_bytes("qs_probe_select_workspace_bytes", B, H, mkbpr)


def qs_probe_select(query, k_cache, block_tables, seq_lens, k, importance=None, n_probe=8,
                    flags=QS_RECENCY, selected=None, n_selected=None, probe_scores=None,
                    workspace_buf=None):
    """Page 1's probe/importance/recency selection per query head.
    Returns (selected [B, H, k] int32, n_selected [B, H] int32)."""
    dev = _dev(query, k_cache, block_tables, seq_lens, importance, selected, n_selected, probe_scores)
    _i32(block_tables, "block_tables")
    _i32(seq_lens, "seq_lens")
    if importance is not None and importance.dtype != torch.float32:
        raise TypeError("importance must be fp32")
    B, H, D = query.shape
    nkv, BS, N, D2 = k_cache.shape
    mkbpr = block_tables.shape[1]
    if selected is None:
        selected = torch.empty((B, H, k), dtype=torch.int32, device=dev)
    if n_selected is None:
        n_selected = torch.empty((B, H), dtype=torch.int32, device=dev)
    _need(D2 == D and H % N == 0, "query and k_cache shapes disagree")
    _rows(block_tables, B, "block_tables")
    _rows(seq_lens, B, "seq_lens")
    _rows(importance, B, "importance")
    _need(selected.numel() >= B * H * k and n_selected.numel() >= B * H, "selected must hold [B, H, k]")
    _need(probe_scores is None or (probe_scores.dtype == torch.float32 and probe_scores.numel() >= B * H * mkbpr),
          "probe_scores must be fp32 [B, H, MKBPR]")
    stride = 0 if importance is None else importance.shape[1]
    nbytes = probe_select_workspace_bytes(B, H, mkbpr)
    st = _stream(dev)
    ws = workspace_buf if workspace_buf is not None else workspace(nbytes, dev, "probe", st)
    _check(lib.qs_probe_select(B, H, N, D, BS, _dtype_code(query), _dtype_code(k_cache), _ptr(query),
                               _ptr(k_cache), nkv, _ptr(block_tables), mkbpr, _ptr(seq_lens), _ptr(importance),
                               stride, int(n_probe), int(k), int(flags), _ptr(selected), _ptr(n_selected),
                               _ptr(probe_scores), _ptr(ws), ws.numel(), st))
    return selected, n_selected


def sparse_attn_workspace_bytes(B, H, N, D, sel_heads, k):
    return _ws_bytes("qs_sparse_attn_workspace_bytes", B, H, N, D, sel_heads, k)


def qs_sparse_attn_decode(query, k_cache, v_cache, block_tables, seq_lens, selected, n_selected,
                          sel_heads=None, k_scale=None, v_scale=None, softmax_scale=0.0, out=None,
                          workspace_buf=None):
    """Exact attention over the selected blocks. Returns out [B, H, D] in the query dtype."""
    dev = _dev(query, k_cache, v_cache, block_tables, seq_lens, selected, n_selected, k_scale, v_scale, out)
    for n, t in (("block_tables", block_tables), ("seq_lens", seq_lens), ("selected", selected),
                 ("n_selected", n_selected)):
        _i32(t, n)
    B, H, D = query.shape
    nkv, BS, N, D2 = k_cache.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must match k_cache")
    if sel_heads is None:
        sel_heads = selected.shape[1]
    k = selected.shape[2]
    _need(D2 == D and H % N == 0, "query and KV shapes disagree")
    _need(selected.dim() == 3 and selected.shape[0] >= B and selected.shape[1] == sel_heads,
          "selected must be [B, sel_heads, k]")
    _need(n_selected.numel() >= B * sel_heads, "n_selected must be [B, sel_heads]")
    _rows(block_tables, B, "block_tables")
    _rows(seq_lens, B, "seq_lens")
    if k_cache.dtype == torch.int8:
        for nm, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
            _need(sc is not None and sc.dtype == torch.float32 and sc.numel() >= nkv * BS * N,
                  f"{nm} must be fp32 [num_kv_blocks, BS, N]")
    if out is None:
        out = torch.empty((B, H, D), dtype=query.dtype, device=dev)
    _need(out.dtype == query.dtype and out.numel() >= B * H * D, "out must be [B, H, D] in the query dtype")
    nbytes = sparse_attn_workspace_bytes(B, H, N, D, sel_heads, k)
    st = _stream(dev)
    ws = workspace_buf if workspace_buf is not None else workspace(nbytes, dev, "attn", st)
    _check(lib.qs_sparse_attn_decode(B, H, N, D, BS, _dtype_code(query), _dtype_code(k_cache), _ptr(query),
                                     _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), nkv,
                                     _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), _ptr(selected),
                                     _ptr(n_selected), int(sel_heads), int(k), float(softmax_scale), _ptr(out),
                                     _ptr(ws), ws.numel(), st))
    return out


def probe_attn_workspace_bytes(B, H, N, mkbpr, k):
    return _ws_bytes("qs_probe_attn_workspace_bytes", B, H, N, mkbpr, k)


def qs_probe_attn_decode(query, k_cache, v_cache, block_tables, seq_lens, k, importance=None, n_probe=8,
                         flags=QS_RECENCY, softmax_scale=0.0, out=None, selected=None, n_selected=None,
                         workspace_buf=None, k_scale=None, v_scale=None, probe_k=None):
    """Page 1's probe selection and attention over it in one call (qs_probe_select then
    qs_sparse_attn_decode with one selection row per query head). Returns out [B, H, D] in
    the query dtype; selected [B, H, k] / n_selected [B, H] receive the selection if given.
    An int8 cache takes its scales (k_scale, v_scale [num_kv_blocks, BS, N] fp32) and the
    float K the probes read (probe_k, paged like k_cache)."""
    dev = _dev(query, k_cache, v_cache, block_tables, seq_lens, importance, out, selected, n_selected, k_scale,
               v_scale, probe_k)
    _i32(block_tables, "block_tables")
    _i32(seq_lens, "seq_lens")
    if importance is not None and importance.dtype != torch.float32:
        raise TypeError("importance must be fp32")
    B, H, D = query.shape
    nkv, BS, N, D2 = k_cache.shape
    mkbpr = block_tables.shape[1]
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must match k_cache")
    _need(D2 == D and H % N == 0, "query and KV shapes disagree")
    q8 = k_cache.dtype == torch.int8
    if q8:
        _need(k_scale is not None and v_scale is not None and probe_k is not None,
              "an int8 cache needs k_scale, v_scale and probe_k")
        _need(k_scale.dtype == v_scale.dtype == torch.float32 and k_scale.shape == v_scale.shape == (nkv, BS, N),
              "k_scale / v_scale must be fp32 [num_kv_blocks, BS, N]")
        _need(probe_k.shape == k_cache.shape and probe_k.dtype != torch.int8, "probe_k must be a float copy of K")
    else:
        _need(k_scale is None and v_scale is None and probe_k is None,
              "k_scale, v_scale and probe_k are for an int8 cache only")
    _rows(block_tables, B, "block_tables")
    _rows(seq_lens, B, "seq_lens")
    _rows(importance, B, "importance")
    _need((selected is None) == (n_selected is None), "selected and n_selected go together")
    if selected is not None:
        _i32(selected, "selected")
        _i32(n_selected, "n_selected")
        _need(selected.numel() >= B * H * k and n_selected.numel() >= B * H, "selected must hold [B, H, k]")
    if out is None:
        out = torch.empty((B, H, D), dtype=query.dtype, device=dev)
    _need(out.dtype == query.dtype and out.numel() >= B * H * D, "out must be [B, H, D] in the query dtype")
    stride = 0 if importance is None else importance.shape[1]
    nbytes = probe_attn_workspace_bytes(B, H, N, mkbpr, k)
    st = _stream(dev)
    ws = workspace_buf if workspace_buf is not None else workspace(nbytes, dev, "probe_attn", st)
    _check(lib.qs_probe_attn_decode(B, H, N, D, BS, _dtype_code(query), _dtype_code(k_cache), _ptr(query),
                                    _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(probe_k),
                                    _dtype_code(probe_k) if q8 else QS_F32, nkv, _ptr(block_tables), mkbpr,
                                    _ptr(seq_lens), _ptr(importance), stride, int(n_probe), int(k), int(flags),
                                    float(softmax_scale), _ptr(out), _ptr(selected), _ptr(n_selected), _ptr(ws),
                                    ws.numel(), st))
    return out


def select_attn_workspace_bytes(B, H, N, block_size, mmbpr, k, dtype):
    return _ws_bytes("qs_select_attn_workspace_bytes", B, H, N, block_size, mmbpr, k, dtype)


def _select_attn_args(query, maxblocks, minblocks, metadata_block_tables, k_cache, v_cache, block_tables,
                      seq_lens, k, tokens_since_update, out, selected, n_selected):
    dev = _dev(query, maxblocks, minblocks, metadata_block_tables, k_cache, v_cache, block_tables, seq_lens,
               tokens_since_update, out, selected, n_selected)
    for n, t in (("metadata_block_tables", metadata_block_tables), ("block_tables", block_tables),
                 ("seq_lens", seq_lens), ("tokens_since_update", tokens_since_update), ("selected", selected),
                 ("n_selected", n_selected)):
        _i32(t, n)
    B, H, D = query.shape
    nmeta, BS, N, D2 = maxblocks.shape
    _need(D2 == D and H % N == 0, "query and metadata shapes disagree")
    _need(maxblocks.shape == minblocks.shape and maxblocks.dtype == minblocks.dtype == query.dtype,
          "maxblocks/minblocks must match each other and the query dtype")
    _need(k_cache.shape[1:] == maxblocks.shape[1:] and v_cache.shape == k_cache.shape and
          k_cache.dtype == v_cache.dtype == query.dtype, "K/V caches must be [num_kv_blocks, BS, N, D] in the query dtype")
    _need((selected is None) == (n_selected is None), "give both selected and n_selected, or neither")
    if selected is not None:
        _need(selected.numel() >= B * N * k and n_selected.numel() >= B * N, "selected must hold [B, N, k]")
    for name, t in (("metadata_block_tables", metadata_block_tables), ("block_tables", block_tables),
                    ("seq_lens", seq_lens), ("tokens_since_update", tokens_since_update)):
        _rows(t, B, name)
    if out is None:
        out = torch.empty((B, H, D), dtype=query.dtype, device=dev)
    _need(out.dtype == query.dtype and out.numel() >= B * H * D, "out must be [B, H, D] in the query dtype")
    return dev, out


def qs_select_attn_decode(query, maxblocks, minblocks, metadata_block_tables, k_cache, v_cache, block_tables,
                          seq_lens, k, tokens_since_update=None, flags=0, softmax_scale=0.0, out=None,
                          selected=None, n_selected=None, workspace_buf=None):
    """Quest selection and attention over the selected blocks in one call (qs_block_select
    then qs_sparse_attn_decode with one selection row per KV head). Returns out [B, H, D];
    pass selected [B, N, k] / n_selected [B, N] to receive the selection too."""
    dev, out = _select_attn_args(query, maxblocks, minblocks, metadata_block_tables, k_cache, v_cache, block_tables,
                                 seq_lens, k, tokens_since_update, out, selected, n_selected)
    B, H, D = query.shape
    nmeta, BS, N, _ = maxblocks.shape
    mmbpr = metadata_block_tables.shape[1]
    dt = _dtype_code(query)
    nbytes = select_attn_workspace_bytes(B, H, N, BS, mmbpr, k, dt)
    st = _stream(dev)
    ws = workspace_buf if workspace_buf is not None else workspace(nbytes, dev, "select_attn", st)
    _check(lib.qs_select_attn_decode(B, H, N, D, BS, dt, _ptr(query), _ptr(maxblocks), _ptr(minblocks), nmeta,
                                     _ptr(metadata_block_tables), mmbpr, _ptr(k_cache), _ptr(v_cache),
                                     k_cache.shape[0], _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens),
                                     _ptr(tokens_since_update), int(flags), int(k), float(softmax_scale), _ptr(out),
                                     _ptr(selected), _ptr(n_selected), _ptr(ws), ws.numel(), st))
    return out


QS_STATIC_SCRATCH_BYTES = 32 << 20


def qs_select_attn_decode_static(query, maxblocks, minblocks, metadata_block_tables, k_cache, v_cache, block_tables,
                                 seq_lens, k, out, tokens_since_update=None, flags=0, softmax_scale=0.0,
                                 selected=None, n_selected=None):
    """qs_select_attn_decode on the library's static device scratch: no workspace, and the
    call allocates nothing (``out``, and the selection outputs if wanted, are the caller's).
    Calls on one GPU share the scratch, so overlapping calls race."""
    _need(out is not None, "out must be given (the call allocates nothing)")
    dev, out = _select_attn_args(query, maxblocks, minblocks, metadata_block_tables, k_cache, v_cache, block_tables,
                                 seq_lens, k, tokens_since_update, out, selected, n_selected)
    B, H, D = query.shape
    nmeta, BS, N, _ = maxblocks.shape
    with torch.cuda.device(dev):
        _check(lib.qs_select_attn_decode_static(B, H, N, D, BS, _dtype_code(query), _ptr(query), _ptr(maxblocks),
                                                _ptr(minblocks), nmeta, _ptr(metadata_block_tables),
                                                metadata_block_tables.shape[1], _ptr(k_cache), _ptr(v_cache),
                                                k_cache.shape[0], _ptr(block_tables), block_tables.shape[1],
                                                _ptr(seq_lens), _ptr(tokens_since_update), int(flags), int(k),
                                                float(softmax_scale), _ptr(out), _ptr(selected), _ptr(n_selected),
                                                _stream(dev)))
    return out


# ---- pool placement ---------------------------------------------------------------------
# The kernels read a head's K and V rows together (and a block's max and min rows) at the
# same offset inside their pools; when the two bases also agree modulo 1 KiB, each pair
# falls in one 256-byte address class, which the chip's memory serves more slowly. These
# helpers place the second pool of a pair 256 bytes past a 1 KiB multiple from the first.

def alloc_paired_pools(shape, dtype, device=None, zero=False):
    """Two contiguous tensors of `shape` (views of one allocation, uninitialised unless
    `zero`), the second starting 256 bytes past a 1 KiB multiple from the first; on the
    current GPU unless `device` is given."""
    if device is None:
        device = torch.device("cuda", torch.cuda.current_device())
    n = 1
    for d in shape:
        n *= int(d)
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    off = (nbytes + 1023) // 1024 * 1024 + 256
    buf = (torch.zeros if zero else torch.empty)(off + nbytes, dtype=torch.uint8, device=device)
    return buf[:nbytes].view(dtype).view(shape), buf[off:off + nbytes].view(dtype).view(shape)


def alloc_kv_pools(num_kv_blocks, block_size, N, D=128, dtype=torch.bfloat16, device=None):
    """k_cache, v_cache [num_kv_blocks, block_size, N, D], uninitialised, placed as the
    header's placement note recommends."""
    return alloc_paired_pools((num_kv_blocks, block_size, N, D), dtype, device)


def alloc_metadata_pools(num_meta_blocks, block_size, N, D=128, dtype=torch.bfloat16, device=None):
    """maxblocks, minblocks [num_meta_blocks, block_size, N, D], zeroed (the +0.0 rows of
    absent blocks), placed as the header's placement note recommends."""
    return alloc_paired_pools((num_meta_blocks, block_size, N, D), dtype, device, zero=True)


def prefill_importance_workspace_bytes(B, H, max_len):
    return _ws_bytes("qs_prefill_importance_workspace_bytes", B, H, max_len)


def prefill_importance_call_workspace_bytes(B, H, max_len, fp32):
    """What one call needs: the full size for fp32 inputs, whose first pass can store the
    scores, else the minimum -- the full size less the stored-score region, which the size
    query adds when B * H * T (T + 1) / 2 tiles of 1 KiB (T = ceil(max_len / 16)) take at
    most 2 GiB."""
    full = prefill_importance_workspace_bytes(B, H, max_len)
    if fp32 or full == 0:
        return full
    t = (max(max_len, 0) + 15) // 16
    scores = B * H * (t * (t + 1) // 2) * 1024
    return full - scores if scores <= (2 << 30) else full


def qs_prefill_importance(query, k_cache, block_tables, seq_lens, softmax_scale=0.0, importance=None,
                          importance_stride=None, head_importance=None, with_heads=False, workspace_buf=None):
    """Page 1's prefill importance from the prefill queries [B, max_len, H, D] and the paged
    K cache. Returns importance [B, stride] fp32 (and head_importance [B, H, stride] when
    with_heads or given)."""
    dev = _dev(query, k_cache, block_tables, seq_lens, importance, head_importance)
    _i32(block_tables, "block_tables")
    _i32(seq_lens, "seq_lens")
    B, max_len, H, D = query.shape
    nkv, BS, N, D2 = k_cache.shape
    _need(D2 == D and H % N == 0 and k_cache.dtype == query.dtype, "query and k_cache shapes/dtypes disagree")
    _rows(block_tables, B, "block_tables")
    _rows(seq_lens, B, "seq_lens")
    stride = importance_stride or (importance.shape[-1] if importance is not None else max(1, max_len))
    if importance is None:
        importance = torch.empty((B, stride), dtype=torch.float32, device=dev)
    _need(importance.dtype == torch.float32 and importance.numel() >= B * stride, "importance must be fp32 [B, stride]")
    if head_importance is None and with_heads:
        head_importance = torch.empty((B, H, stride), dtype=torch.float32, device=dev)
    if head_importance is not None:
        _need(head_importance.dtype == torch.float32 and head_importance.numel() >= B * H * stride,
              "head_importance must be fp32 [B, H, stride]")
    nbytes = prefill_importance_call_workspace_bytes(B, H, max_len, query.dtype == torch.float32)
    st = _stream(dev)
    ws = workspace_buf if workspace_buf is not None else workspace(nbytes, dev, "importance", st)
    _check(lib.qs_prefill_importance(B, H, N, D, BS, _dtype_code(query), _ptr(query), max_len, _ptr(k_cache), nkv,
                                     _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), float(softmax_scale),
                                     _ptr(importance), int(stride), _ptr(head_importance), _ptr(ws), ws.numel(),
                                     st))
    return (importance, head_importance) if head_importance is not None else importance
