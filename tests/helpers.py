"""Test-side helpers: marshalling only (gathering paged rows, reading fixtures,
comparing selections under the near-tie rule). None of the method's arithmetic."""

from __future__ import annotations

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


def cdiv(a, b):
    return -(-a // b)


def f64(x):
    """float64 numpy copy of a CPU/GPU torch tensor (bf16 widened exactly)."""
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().float().double().numpy()
    return np.asarray(x, dtype=np.float64)


def request_tokens(wl, b, kind="k"):
    """[L, N, D] float64 rows of request b in sequence order (through block_tables)."""
    cache = wl.k_cache if kind == "k" else wl.v_cache
    L = int(wl.seq_lens[b])
    nb = cdiv(L, wl.BS)
    phys = wl.block_tables[b, :nb].long().cpu()
    rows = cache.cpu()[phys].reshape(nb * wl.BS, wl.N, wl.D)[:L]
    return f64(rows)


def block_rows(wl, b, i, kind="k", cover=None):
    """[nt, N, D] float64 rows of sequence-relative block i of request b (valid tokens)."""
    L = int(wl.seq_lens[b] if cover is None else cover)
    cache = wl.k_cache if kind == "k" else wl.v_cache
    phys = int(wl.block_tables[b, i])
    nt = min(wl.BS, L - i * wl.BS)
    return f64(cache.cpu()[phys, :nt])


def as_sets(selected, n_selected):
    """List of python sets of the valid indices per row (flattened rows)."""
    sel = np.asarray(selected).reshape(-1, np.asarray(selected).shape[-1])
    ns = np.asarray(n_selected).reshape(-1)
    return [set(int(x) for x in sel[r, :ns[r]]) for r in range(sel.shape[0])]


def check_selection_rows(selected, n_selected, k):
    """Structural validity: ascending, unique, -1 padded, count = n_selected."""
    sel = np.asarray(selected).reshape(-1, k)
    ns = np.asarray(n_selected).reshape(-1)
    for r in range(sel.shape[0]):
        n = int(ns[r])
        assert 0 <= n <= k
        v = sel[r, :n]
        assert np.all(v >= 0)
        assert np.all(np.diff(v) > 0), f"row {r} not strictly ascending: {v}"
        assert np.all(sel[r, n:] == -1), f"row {r} padding: {sel[r]}"


def near_tie_equal(got, want, fill_scores, fixed, rel=1e-3):
    """Near-tie rule for one selection row.

    got, want: sets of indices; fixed: indices the rule requires exactly (forced or
    importance picks, which must always match); fill_scores: dict index -> oracle
    fill-stage score for every fill candidate. Let s_k / s_k1 be the oracle's lowest
    selected and highest unselected fill scores. If the gap exceeds rel*|s_k| the sets
    must be equal; otherwise they may differ only in blocks whose oracle score is within
    rel*|s_k| of s_k.
    """
    if not fixed <= got:
        return False, f"fixed picks {sorted(fixed - got)} missing"
    if len(got) != len(want):
        return False, f"sizes differ {len(got)} vs {len(want)}"
    if got == want:
        return True, ""
    fill_want = want - fixed
    if not fill_want:
        return False, "no fill picks in oracle yet sets differ"
    s_k = min(fill_scores[i] for i in fill_want)
    tol = rel * max(abs(s_k), 1e-30)
    for i in (got ^ want):
        if i not in fill_scores:
            return False, f"index {i} is not a fill candidate"
        if abs(fill_scores[i] - s_k) > tol:
            return False, f"index {i} score {fill_scores[i]} not within {tol} of s_k={s_k}"
    return True, "near tie"
