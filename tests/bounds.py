"""Error bound of the 16-bit matrix-core attention against the oracle's float64 output.

Test infrastructure: it sizes the tolerance of a comparison, it is never the reference.
The reference output always comes from the oracle; this module recomputes the softmax
weights of the selected tokens in float64 only to size the bound of each output element.

What the matrix-core attention does to a head's weights (16-bit query and KV):

* the logits q.k are accumulated in fp32 from exactly widened 16-bit values, scaled by
  scale*log2(e) and exponentiated with the hardware exp2 (relative error ~2^-22);
* each unnormalised weight p_t (relative to the running maximum, so p_t <= 1) is rounded
  to the operand format before the P.V product, and the denominator sums the *rounded*
  weights: p~_t = p_t (1 + d_t) (+ e_t, an absolute error <= 2^-25 when fp16 turns p_t
  subnormal), |d_t| <= u_P, with u_P = 2^-8 (bf16) or 2^-11 (fp16);
* the products and sums are accumulated in fp32, split partials merged with fp32
  rescales, and the output is rounded once to the query dtype (relative error u_O).

With normalised weights w_t = p_t / sum p, exact algebra gives for output element d

    out~_d - out_d = sum_t w_t d_t (V_td - out_d) / (1 + sum_s w_s d_s).

The worst case (all d_t aligned with the sign of V_td - out_d) is u_P sum_t w_t |V_td - out_d|,
which over thousands of tokens is two orders of magnitude above what any correct kernel
shows and wide enough to hide a dropped block. The bound used here takes the standard
statistical model of rounding (independent, zero-mean errors bounded by their unit
roundoff; Higham, "Accuracy and Stability of Numerical Algorithms", section 2.8) and
Hoeffding's inequality, P(|sum a_t d_t| > z sqrt(sum a_t^2 u_t^2)) <= 2 exp(-z^2 / 2). With
z = 7 that is 5e-11 per element, so a correct kernel passes on millions of elements:

    tol_d = u_O |out_d|
          + (1 + u_O) [ 7 sqrt(sum_t w_t^2 u_t^2 (V_td - out_d)^2)                (P rounding)
                      + 7 * 2^-25 w_max sqrt(sum_t (V_td - out_d)^2)   (fp16 subnormals only)
                      + (7 sqrt(n) + 8) 2^-24 (sum_t w_t |V_td| + |out_d|) ]    (fp32 sums)

where u_t = u_P + ln2 * eta_t + 2^-22 per token, eta_t bounds the fp32 logit error in
base-2 units: 2^-24 (132 |s2| sum_d |q_d k_td| + 2 |l_t| + 2 |l_t - l_max|), s2 = scale *
log2(e), l_t = s2 q.k_t. n is the number of attended tokens. Every term is computed from
the inputs; nothing is fitted to the kernel's observed errors.
"""

from __future__ import annotations

import math

import numpy as np
import torch

LOG2E = 1.0 / math.log(2.0)
Z = 7.0


def _f64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _raw16(t):
    """numpy view of a CPU 16-bit torch tensor's bit patterns (no copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _widen16(bits, dtype):
    """Exact float64 values of bf16 / fp16 bit patterns."""
    if dtype == torch.bfloat16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def unit_roundoff(dtype) -> float:
    return {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}[dtype]


def row_tokens(block_tables, seq_len, sel_row, BS):
    """(physical block, first token, valid tokens) of each entry of one selection row,
    in entry order, skipping entries the attention skips (negative or past the blocks)."""
    L = max(int(seq_len), 0)
    nb = -(-L // BS)
    out = []
    for blk in sel_row:
        blk = int(blk)
        if blk < 0 or blk >= nb or blk >= block_tables.shape[0]:
            continue
        out.append((int(block_tables[blk]), blk * BS, min(BS, L - blk * BS)))
    return out


def attn16_bound(query, k_cache, v_cache, block_tables, seq_lens, selected, n_selected, sel_heads, ref,
                 dtype, softmax_scale=0.0):
    """Per-element tolerance [B, H, D] of the matrix-core attention output (in ``dtype``,
    bf16 or fp16) against the oracle's float64 ``ref`` over the same selection."""
    q = _f64(query)
    B, H, D = q.shape
    kc, vc = _raw16(k_cache), _raw16(v_cache)
    N, BS = kc.shape[2], kc.shape[1]
    bt = np.asarray(block_tables.cpu() if isinstance(block_tables, torch.Tensor) else block_tables)
    sl = np.asarray(seq_lens.cpu() if isinstance(seq_lens, torch.Tensor) else seq_lens)
    sel = np.asarray(selected.cpu() if isinstance(selected, torch.Tensor) else selected)
    ns = np.asarray(n_selected.cpu() if isinstance(n_selected, torch.Tensor) else n_selected)
    ref = np.asarray(ref, dtype=np.float64)
    scale = softmax_scale if softmax_scale > 0 else 1.0 / math.sqrt(D)
    s2 = scale * LOG2E
    uP = unit_roundoff(dtype)
    uO = uP
    sub = 2.0 ** -25 if dtype == torch.float16 else 0.0
    G = H // N
    hpr = H // sel_heads
    tol = np.zeros((B, H, D), np.float64)
    for b in range(B):
        for s in range(sel_heads):
            h0 = s * hpr
            kh = h0 // G
            ents = row_tokens(bt[b], sl[b], sel[b, s, :max(0, min(int(ns[b, s]), sel.shape[-1]))], BS)
            outs = ref[b, h0:h0 + hpr]                                   # [hpr, D]
            if not ents:
                continue
            phys = np.array([e[0] for e in ents], dtype=np.int64)
            keep = np.concatenate([np.arange(e[2]) + i * BS for i, e in enumerate(ents)])
            K = _widen16(kc[phys, :, kh].reshape(-1, D)[keep], dtype)     # [T, D]
            V = _widen16(vc[phys, :, kh].reshape(-1, D)[keep], dtype)
            qs = q[b, h0:h0 + hpr]                                       # [hpr, D]
            lg = s2 * (qs @ K.T)                                         # [hpr, T] base-2 logits
            lmax = lg.max(axis=1, keepdims=True)
            w = np.exp2(lg - lmax)
            w /= w.sum(axis=1, keepdims=True)
            eta = 2.0 ** -24 * (132.0 * abs(s2) * (np.abs(qs) @ np.abs(K).T) + 2.0 * np.abs(lg)
                                + 2.0 * np.abs(lg - lmax))
            u = uP + math.log(2.0) * eta + 2.0 ** -22                    # [hpr, T]
            # sum_t c_t (V_td - out_d)^2 expanded into products with V and V^2 (float64)
            V2 = V * V

            def spread(c):
                return np.maximum(c @ V2 - 2.0 * outs * (c @ V) + outs * outs * c.sum(axis=1, keepdims=True), 0.0)

            r = np.sqrt(spread((w * u) ** 2))
            rs = sub * w.max(axis=1, keepdims=True) * np.sqrt(spread(np.ones_like(w))) if sub else 0.0
            a = w @ np.abs(V)
            n = K.shape[0]
            acc = (Z * math.sqrt(n) + 8.0) * 2.0 ** -24 * (a + np.abs(outs))
            tol[b, h0:h0 + hpr] = uO * np.abs(outs) + (1.0 + uO) * (Z * r + Z * rs + acc)
    return tol


def check_attn16(got, ref, tol, what, contract=2e-2, log=print):
    """Asserts |got - ref| <= tol element-wise and <= ``contract`` (the absolute tolerance
    of the contract); logs the largest error and the largest error/tolerance ratio."""
    g = _f64(got)
    err = np.abs(g - ref)
    ratio = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    log(f"{what}: max abs err {float(err.max()) if err.size else 0.0:.3e} (contract {contract:g}), "
        f"max err/bound {ratio:.3f}, median bound {float(np.median(tol)) if tol.size else 0.0:.2e}")
    assert err.size == 0 or float(err.max()) <= contract, f"{what}: max abs err {float(err.max()):.3e} > {contract}"
    bad = np.argwhere(err > tol)
    assert bad.size == 0, (f"{what}: {len(bad)} elements beyond the rounding bound, first {tuple(bad[0])}: "
                           f"err {err[tuple(bad[0])]:.3e} > bound {tol[tuple(bad[0])]:.3e}")
    return ratio
