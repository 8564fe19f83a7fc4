"""Seeded synthetic inputs for the sparse-decode path.

This module only *makes inputs*: random tensors, paged block tables, sequence lengths,
planted "needle" keys and the int8 copies of a KV cache. It computes none of the
path's own steps (no metadata, scores, selection or attention), so both the HIP path
and the CPU oracle can take their inputs from here without sharing any arithmetic.

Shapes follow the two pages' workloads:

* page 3 ("ops-transformer select_attention_operators", usage example and the
  "quest_prefill_metadata" example): paged KV cache ``[num_kv_blocks, BS, N, D]``,
  ``block_tables [B, MKBPR]`` and ``metadata_block_tables [B, MMBPR]`` holding random
  permutations, BS = D = 128;
* page 1 ("0.8MB runs Qwen 10-2", section 2): 32-token blocks, 8 probes per block,
  per-token prefill importance, an fp32 KV cache with an int8 copy.

Small cases are drawn on the CPU (identical on every machine). The large cases
(the page-3 example, long-context and serving workloads below) are drawn on the device the caller names, with a seeded
``torch.Generator`` there, and copied to the host when the oracle needs them.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# flag bits of the selection calls (same values as the C header)
FORCE_SINK = 1
FORCE_WINDOW = 2
RECENCY = 4


@dataclasses.dataclass
class Workload:
    """One batch of decode-step inputs. Tensors live on ``device``."""

    name: str
    B: int
    H: int
    N: int
    D: int
    BS: int
    k: int
    query: torch.Tensor                      # [B, H, D]
    k_cache: torch.Tensor                    # [num_kv_blocks, BS, N, D]
    v_cache: Optional[torch.Tensor]          # same shape as k_cache, or None (select-only)
    block_tables: torch.Tensor               # [B, MKBPR] int32, physical KV block ids
    seq_lens: torch.Tensor                   # [B] int32, tokens in each request
    meta_tables: torch.Tensor                # [B, MMBPR] int32, physical metadata block ids
    num_meta_blocks: int
    meta_seq_lens: torch.Tensor              # [B] int32, tokens covered by the metadata
    tsmu: Optional[torch.Tensor] = None      # [B] int32 tokens since the metadata update
    flags: int = 0
    sel_heads: int = 0                       # selection rows per request (N or H)
    n_probe: int = 8
    importance: Optional[torch.Tensor] = None  # [B, max_seq] fp32
    k_i8: Optional[torch.Tensor] = None      # int8 copy of k_cache
    v_i8: Optional[torch.Tensor] = None
    k_scale: Optional[torch.Tensor] = None   # [num_kv_blocks, BS, N] fp32
    v_scale: Optional[torch.Tensor] = None
    needles: Optional[list] = None           # [(b, token)] planted needle positions
    extra: dict = dataclasses.field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.H // self.N

    @property
    def mkbpr(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def mmbpr(self) -> int:
        return int(self.meta_tables.shape[1])

    @property
    def num_kv_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    def to(self, device) -> "Workload":
        """A copy with every tensor moved to ``device``."""
        out = dataclasses.replace(self)
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            if isinstance(v, torch.Tensor):
                setattr(out, f.name, v.to(device))
        return out


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _uniform(shape, g, device, lo=-1.0, hi=1.0):
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def _normal(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def paired_pools(shape, dtype, device):
    """Two uninitialised contiguous tensors of `shape` in one allocation, the second starting
    256 bytes past a 1 KiB multiple from the first: the placement the library documents for
    a K / V pool pair (a head's K and V rows then fall in different 256-byte address
    classes). The large paged workloads are laid out this way, as a caller following the
    library's placement note would allocate them."""
    n = 1
    for d in shape:
        n *= int(d)
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    off = (nbytes + 1023) // 1024 * 1024 + 256
    buf = torch.empty(off + nbytes, dtype=torch.uint8, device=device)
    return buf[:nbytes].view(dtype).view(shape), buf[off:off + nbytes].view(dtype).view(shape)


def _fill_blocks(n_blocks, BS, N, D, g, device, dist, dtype, chunk_blocks=1024, out=None):
    """A KV pool drawn block-chunk by block-chunk (keeps the fp32 temporary small), into
    `out` when given."""
    if out is None:
        out = torch.empty((n_blocks, BS, N, D), dtype=dtype, device=device)
    for s in range(0, n_blocks, chunk_blocks):
        e = min(n_blocks, s + chunk_blocks)
        shape = (e - s, BS, N, D)
        x = _uniform(shape, g, device) if dist == "uniform" else _normal(shape, g, device)
        out[s:e].copy_(x.to(dtype))
    return out


def quantize_rows_int8(x: torch.Tensor):
    """int8 copy of a KV pool: one scale per (token, kv-head) row of D values.

    scale = absmax / 127; code = clamp(round-half-even(x / scale), -127, 127);
    an all-zero row gets scale 0 and codes 0. Done in fp32.
    """
    x = x.float()
    amax = x.abs().amax(dim=-1)
    scale = amax / 127.0
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    q = torch.round(x / safe.unsqueeze(-1))           # torch.round is half-to-even
    q = torch.clamp(q, -127, 127)
    q = torch.where(scale.unsqueeze(-1) > 0, q, torch.zeros_like(q))
    return q.to(torch.int8), scale.contiguous()


def _paged_tables(nbs, g, device, capacity=None):
    """Block tables for requests with ``nbs[b]`` blocks, sliced from one random
    permutation of a pool of sum(nbs) physical blocks; unused slots hold 0."""
    total = int(sum(nbs))
    cap = int(capacity if capacity is not None else max(nbs))
    perm = torch.randperm(total, generator=g, device=device).to(torch.int32)
    tables = torch.zeros((len(nbs), cap), dtype=torch.int32, device=device)
    off = 0
    for b, nb in enumerate(nbs):
        tables[b, :nb] = perm[off:off + nb]
        off += nb
    return tables, total


def _cdiv(a, b):
    return -(-a // b)


# ----------------------------------------------------------------------------------------
# the five benchmark / parity configurations
# ----------------------------------------------------------------------------------------

def tiny_needle(seed: int = 0) -> Workload:
    """Tiny Quest select + sparse attention, fp32 (CPU-drawn).

    B=1, H=4, N=1, D=128, BS=32, seq_len=2048 (64 blocks), k=8. Query, K and V are
    i.i.d. U(-1,1); the key at token 1000 is replaced by 4x the mean of the request's
    query heads (the needle). Contiguous block table; metadata spans 2 metadata blocks.
    """
    B, H, N, D, BS, L, k = 1, 4, 1, 128, 32, 2048, 8
    g = _gen(seed, "cpu")
    nb = L // BS
    q = _uniform((B, H, D), g, "cpu")
    kc = _uniform((nb, BS, N, D), g, "cpu")
    vc = _uniform((nb, BS, N, D), g, "cpu")
    t = 1000
    kc[t // BS, t % BS, 0, :] = 4.0 * q[0].mean(dim=0)
    bt = torch.arange(nb, dtype=torch.int32).reshape(1, nb)
    mmbpr = _cdiv(nb, BS)
    mt = torch.arange(mmbpr, dtype=torch.int32).reshape(1, mmbpr)
    sl = torch.full((B,), L, dtype=torch.int32)
    return Workload("tiny_b1_h4_l2048_fp32", B, H, N, D, BS, k, q, kc, vc, bt, sl, mt, mmbpr,
                    sl.clone(), tsmu=None, flags=0, sel_heads=N, needles=[(0, t)])


def page3_select(device="cpu", seed: int = 1, B: int = 20, nb: int = 128, dtype=torch.bfloat16) -> Workload:
    """Quest select shaped like page 3's usage example, bf16 (or ``dtype``, e.g. fp16).

    B=20, H=32, N=8, D=128, BS=128, MMBPR=1, seq_len=16384 (128 blocks), k=8.
    K ~ U(-1,1) in a pool of B*128 physical blocks with a random-permutation block
    table; metadata blocks also a random permutation; query U(-1,1). No V (select only).
    ``B`` and ``nb`` can be reduced for CPU-sized parity cases.
    """
    H, N, D, BS, k = 32, 8, 128, 128, 8
    L = nb * BS
    g = _gen(seed, device)
    n_kv = B * nb
    kc = _fill_blocks(n_kv, BS, N, D, g, device, "uniform", dtype)
    bt = torch.randperm(n_kv, generator=g, device=device).to(torch.int32).reshape(B, nb)
    mmbpr = _cdiv(nb, BS)
    n_meta = B * mmbpr
    mt = torch.randperm(n_meta, generator=g, device=device).to(torch.int32).reshape(B, mmbpr)
    q = _uniform((B, H, D), g, device).to(dtype)
    sl = torch.full((B,), L, dtype=torch.int32, device=device)
    name = {torch.bfloat16: "bf16", torch.float16: "fp16"}.get(dtype, str(dtype))
    return Workload(f"page3_select_b{B}_l{L}_{name}", B, H, N, D, BS, k, q, kc, None, bt, sl, mt,
                    n_meta, sl.clone(), tsmu=None, flags=0, sel_heads=N)


def page1_probe(seed: int = 3, k: int = 32) -> Workload:
    """Page 1's probe selection, fp32 with an int8 copy (CPU-drawn).

    B=1, H=16, N=8 (group 2), D=128, BS=32, seq_len=4096 (128 blocks), n_probe=8.
    K, V ~ N(0,1) fp32, contiguous table; int8 copies with per-(token, kv-head) absmax
    scales. Query ~ N(0,1). At token 2000 every kv-head's key is sqrt(D) times the
    unit vector of the mean of its two query heads (the needle). Prefill importance:
    0.5 * Dirichlet(0.1 * ones(4096)) + 0.5 * uniform mass on the last 256 tokens.
    Recency on; selection per query head, so attention takes sel_heads = H.
    """
    B, H, N, D, BS, L = 1, 16, 8, 128, 32, 4096
    g = _gen(seed, "cpu")
    nb = L // BS
    q = _normal((B, H, D), g, "cpu")
    kc = _normal((nb, BS, N, D), g, "cpu")
    vc = _normal((nb, BS, N, D), g, "cpu")
    t = 2000
    G = H // N
    for kh in range(N):
        m = q[0, kh * G:(kh + 1) * G].mean(dim=0)
        kc[t // BS, t % BS, kh, :] = math.sqrt(D) * m / m.norm()
    rng = np.random.default_rng(seed)
    imp = 0.5 * rng.dirichlet(np.full(L, 0.1))
    imp[L - 256:] += 0.5 / 256.0
    importance = torch.from_numpy(imp.astype(np.float32)).reshape(B, L)
    k8, ks = quantize_rows_int8(kc)
    v8, vs = quantize_rows_int8(vc)
    bt = torch.arange(nb, dtype=torch.int32).reshape(1, nb)
    mt = torch.zeros((1, 1), dtype=torch.int32)
    sl = torch.full((B,), L, dtype=torch.int32)
    return Workload("page1_probe_b1_h16_l4096_fp32_int8", B, H, N, D, BS, k, q, kc, vc, bt, sl, mt, 1,
                    sl.clone(), tsmu=None, flags=RECENCY, sel_heads=H, n_probe=8,
                    importance=importance, k_i8=k8, v_i8=v8, k_scale=ks, v_scale=vs,
                    needles=[(0, t)])


def long_context(device="cpu", seed: int = 2, B: int = 8, min_len: int = 8192,
            max_len: int = 131072) -> Workload:
    """Long-context paged decode, bf16.

    B=8, H=32, N=8, D=128, BS=128, k=64. seq_len_b ~ U{8192..131072} (up to 1024 blocks,
    8 metadata blocks). K, V ~ N(0,1) in one pool of sum(blocks) physical blocks sliced
    from one random permutation. One needle per request: a token drawn uniformly in
    the middle half of its blocks whose key for kv-head n is 4*sqrt(D) times the unit
    vector of the mean of that group's query heads. tokens_since_metadata_update =
    seq_len mod 128, metadata built over seq_len - tsmu tokens; sink + window forcing.
    """
    H, N, D, BS, k = 32, 8, 128, 128, 64
    g = _gen(seed, device)
    sl = torch.randint(min_len, max_len + 1, (B,), generator=g, device=device,
                       dtype=torch.int64).to(torch.int32)
    sl_h = sl.cpu().tolist()
    nbs = [_cdiv(L, BS) for L in sl_h]
    mkbpr = _cdiv(max_len, BS)
    bt, n_kv = _paged_tables(nbs, g, device, capacity=mkbpr)
    kc, vc = paired_pools((n_kv, BS, N, D), torch.bfloat16, device)
    _fill_blocks(n_kv, BS, N, D, g, device, "normal", torch.bfloat16, out=kc)
    _fill_blocks(n_kv, BS, N, D, g, device, "normal", torch.bfloat16, out=vc)
    q = _normal((B, H, D), g, device).to(torch.bfloat16)
    mnbs = [_cdiv(nb, BS) for nb in nbs]
    mmbpr = _cdiv(mkbpr, BS)
    mt, n_meta = _paged_tables(mnbs, g, device, capacity=mmbpr)
    tsmu = (sl % BS).to(torch.int32)
    msl = (sl - tsmu).to(torch.int32)
    needles = []
    G = H // N
    bt_h = bt.cpu()
    for b in range(B):
        nb = nbs[b]
        lo, hi = (nb // 4) * BS, max((3 * nb // 4) * BS, (nb // 4) * BS + 1)
        t = int(torch.randint(lo, hi, (1,), generator=g, device=device).item())
        needles.append((b, t))
        qb = q[b].float().reshape(N, G, D).mean(dim=1)            # [N, D]
        dirn = qb / qb.norm(dim=-1, keepdim=True)
        phys = int(bt_h[b, t // BS])
        kc[phys, t % BS] = (4.0 * math.sqrt(D) * dirn).to(torch.bfloat16)
    return Workload(f"long_context_b{B}_l{min_len // 1024}k_{max_len // 1024}k_bf16", B, H, N, D, BS, k, q, kc, vc, bt, sl, mt,
                    n_meta, msl, tsmu=tsmu, flags=FORCE_SINK | FORCE_WINDOW, sel_heads=N,
                    needles=needles)


def serving(device="cpu", seed: int = 4, B: int = 128, nb: int = 256,
            n_query_sets: int = 4) -> Workload:
    """Large-batch serving decode, bf16.

    B=128, H=64, N=8 (group 8), D=128, BS=128, seq_len=32768 (256 blocks), k=16.
    K, V ~ N(0,1) in a pool of B*256 physical blocks (8 GiB each at full size) with a
    shuffled block table; metadata tables shuffled too. ``n_query_sets`` independent
    query sets ~ N(0,1) are drawn (``extra['query_sets']``, [R, B, H, D]) so that
    consecutive steps select different blocks. Sink + window forcing; step s uses
    tokens_since_metadata_update = s mod 128 with seq_len held fixed.
    """
    H, N, D, BS, k = 64, 8, 128, 128, 16
    L = nb * BS
    g = _gen(seed, device)
    n_kv = B * nb
    bt = torch.randperm(n_kv, generator=g, device=device).to(torch.int32).reshape(B, nb)
    kc, vc = paired_pools((n_kv, BS, N, D), torch.bfloat16, device)
    _fill_blocks(n_kv, BS, N, D, g, device, "normal", torch.bfloat16, out=kc)
    _fill_blocks(n_kv, BS, N, D, g, device, "normal", torch.bfloat16, out=vc)
    qs = _normal((n_query_sets, B, H, D), g, device).to(torch.bfloat16)
    mmbpr = _cdiv(nb, BS)
    n_meta = B * mmbpr
    mt = torch.randperm(n_meta, generator=g, device=device).to(torch.int32).reshape(B, mmbpr)
    sl = torch.full((B,), L, dtype=torch.int32, device=device)
    tsmu = torch.zeros((B,), dtype=torch.int32, device=device)
    return Workload(f"serving_b{B}_h{H}_l{L}_bf16", B, H, N, D, BS, k, qs[0].contiguous(), kc, vc, bt,
                    sl, mt, n_meta, sl.clone(), tsmu=tsmu, flags=FORCE_SINK | FORCE_WINDOW,
                    sel_heads=N, extra={"query_sets": qs})


def extra_queries(wl: Workload, seed: int) -> torch.Tensor:
    """An independent query set ~ N(0,1) for ``wl``'s requests, [B, H, D] in the query dtype,
    drawn on the workload's device (a later decode step's queries on the same KV pools)."""
    device = wl.query.device
    return _normal((wl.B, wl.H, wl.D), _gen(seed, device), device).to(wl.query.dtype)


# ----------------------------------------------------------------------------------------
# small randomised cases for parity sweeps
# ----------------------------------------------------------------------------------------

def random_case(seed: int, B: int, H: int, N: int, BS: int, seq_lens, k: int,
                dtype=torch.float32, D: int = 128, dist: str = "normal",
                meta_cover=None, tsmu=None, flags: int = 0, sel_heads: int = 0,
                with_v: bool = True, with_importance: bool = False, n_probe: int = 8,
                int8: bool = False, spare_blocks: int = 3, meta_spare: int = 2) -> Workload:
    """A small paged case on the CPU with ragged lengths and shuffled tables.

    ``seq_lens`` may hold zeros and partial blocks. The pools carry ``spare_blocks``
    extra physical blocks (never referenced) so that a wrong table lookup reads a
    block that is not part of the request. ``meta_cover[b]`` (default seq_lens) is the
    number of tokens the metadata is built over.
    """
    g = _gen(seed, "cpu")
    seq_lens = [int(x) for x in seq_lens]
    nbs = [_cdiv(L, BS) for L in seq_lens]
    mkbpr = max(1, max(nbs))
    n_kv = sum(nbs) + spare_blocks
    perm = torch.randperm(n_kv, generator=g).to(torch.int32)
    bt = torch.zeros((B, mkbpr), dtype=torch.int32)
    off = 0
    for b, nb in enumerate(nbs):
        bt[b, :nb] = perm[off:off + nb]
        off += nb
    draw = _uniform if dist == "uniform" else (lambda s, gg, d: _normal(s, gg, d))
    kc = draw((n_kv, BS, N, D), g, "cpu").to(dtype)
    vc = draw((n_kv, BS, N, D), g, "cpu").to(dtype) if with_v else None
    q = draw((B, H, D), g, "cpu").to(dtype)
    mnbs = [max(1, _cdiv(nb, BS)) for nb in nbs]
    mmbpr = max(mnbs)
    n_meta = sum(mnbs) + meta_spare
    mperm = torch.randperm(n_meta, generator=g).to(torch.int32)
    mt = torch.zeros((B, mmbpr), dtype=torch.int32)
    off = 0
    for b, mnb in enumerate(mnbs):
        mt[b, :mnb] = mperm[off:off + mnb]
        off += mnb
    sl = torch.tensor(seq_lens, dtype=torch.int32)
    msl = torch.tensor(meta_cover if meta_cover is not None else seq_lens, dtype=torch.int32)
    ts = None if tsmu is None else torch.tensor(tsmu, dtype=torch.int32)
    importance = None
    if with_importance:
        maxL = max(1, max(seq_lens))
        importance = torch.rand((B, maxL), generator=g, dtype=torch.float32)
    wl = Workload(f"random_{seed}", B, H, N, D, BS, k, q, kc, vc, bt, sl, mt, n_meta, msl,
                  tsmu=ts, flags=flags, sel_heads=sel_heads or N, n_probe=n_probe,
                  importance=importance)
    if int8:
        wl.k_i8, wl.k_scale = quantize_rows_int8(kc.float())
        wl.v_i8, wl.v_scale = quantize_rows_int8(vc.float())
    return wl


def prefill_queries(wl: Workload, seed: int, max_len: int = 0, dist: str = "normal") -> torch.Tensor:
    """Prefill query rows for ``wl``'s requests: [B, max_len, H, D] in the workload's float
    dtype (fp32 for an int8 workload), drawn on the workload's device. ``max_len``
    defaults to the longest request. Rows past a request's length are drawn too (unused)."""
    device = wl.k_cache.device
    L = max_len or max(1, int(wl.seq_lens.max()))
    g = _gen(seed, device)
    x = _uniform((wl.B, L, wl.H, wl.D), g, device) if dist == "uniform" else _normal((wl.B, L, wl.H, wl.D), g, device)
    dt = wl.k_cache.dtype if wl.k_cache.dtype != torch.int8 else torch.float32
    return x.to(dt)


def page1_probe_prefill(seed: int = 5):
    """The prefill that produces page 1's importance for the page-1 probe workload: its requests and
    K cache (B=1, H=16, N=8, D=128, BS=32, 4096 tokens, fp32) with 4096 prefill query rows
    ~ N(0,1). Returns (workload, queries [1, 4096, 16, 128])."""
    wl = page1_probe()
    return wl, prefill_queries(wl, seed)
