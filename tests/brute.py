"""Brute-force routes to the oracle's results, for tiny inputs only.

Each helper reaches the same quantity as the oracle by a different road, so
that a slip in the oracle (an index, a sign, a dropped term, a transposed
operand) shows up as a mismatch:

* scores through the raw tokens, using the linearity of the pooled dot
  product (q . mean_r k_r = mean_r q . k_r, and likewise for a gate-weighted
  sum) rather than a pooled key table;
* selection by counting ranks (p is kept iff fewer than k pools beat it,
  where beating means a larger fp32 score or an equal one at a lower id),
  not by sorting;
* attention through torch's scaled_dot_product_attention in float64 with an
  explicit boolean mask.
"""
from __future__ import annotations

import numpy as np
import torch


def bf16_to_f64(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.float64).numpy()


def raw_token_scores(q_idx, k_idx, w, q_pos0=0, rows=None, pool=4, gate=None) -> np.ndarray:
    """fp32 scores [len(rows), P] via raw tokens; -inf for ineligible pools.
    With per-token gates [S_k] the pooled dot is sum_r g_r (q . k_r) instead of
    the mean."""
    q = bf16_to_f64(q_idx)              # [S_q, H, D]
    k = bf16_to_f64(k_idx)              # [S_k, D]
    gv = None if gate is None else np.asarray(gate, dtype=np.float32).astype(np.float64)
    wv = w.to(torch.float64).numpy()
    s_q = q.shape[0]
    n_pools = k.shape[0] // pool
    rows = np.arange(s_q) if rows is None else np.asarray(rows)
    out = np.full((len(rows), n_pools), -np.inf, dtype=np.float32)
    for a, i in enumerate(rows):
        t = q_pos0 + int(i)
        n = min(t // pool, n_pools)
        if n == 0:
            continue
        toks = k[: n * pool]                       # [n*pool, D]
        per_tok = q[i] @ toks.T                    # [H, n*pool]
        if gv is None:
            pooled = per_tok.reshape(q.shape[1], n, pool).mean(axis=2)   # [H, n]
        else:
            pooled = (per_tok * gv[None, : n * pool]).reshape(q.shape[1], n, pool).sum(axis=2)
        wr = wv if wv.ndim == 1 else wv[i]
        s = (wr[:, None] * np.maximum(pooled, 0.0)).sum(axis=0)
        s32 = s.astype(np.float32)
        s32[s32 == 0] = 0.0
        out[a, :n] = s32
    return out


def rank_select(scores_row: np.ndarray, n: int, k: int) -> np.ndarray:
    """Pool ids kept by rank counting, ascending, -1 padded to k."""
    s = scores_row[:n].astype(np.float32)
    kept = []
    for p in range(n):
        beaten_by = np.count_nonzero(s > s[p]) + np.count_nonzero(s[:p] == s[p])
        if beaten_by < k:
            kept.append(p)
    kept = kept + [-1] * (k - len(kept))
    return np.array(kept, dtype=np.int32)


def dense_attention(q, k, v, q_pos0, rows, include_own_prefix: bool, scale: float,
                    pool=4):
    """Masked dense attention through torch SDPA (float64).

    Token j is visible to the query at position t iff j < pool*floor(t/pool)
    (every earlier complete pool), or iff j < t when ``include_own_prefix``.
    Returns (o [len(rows), H, Dv], lse [len(rows), H]); rows with no visible
    token come back as NaN from SDPA and are left to the caller."""
    qf = q.to(torch.float64)
    kf = k.to(torch.float64)
    vf = v.to(torch.float64)
    s_k = kf.shape[0]
    rows = list(int(r) for r in rows)
    pos = torch.tensor([q_pos0 + r for r in rows])
    j = torch.arange(s_k)
    if include_own_prefix:
        mask = j[None, :] < pos[:, None]
    else:
        mask = j[None, :] < (pos[:, None] // pool) * pool
    qs = qf[rows].permute(1, 0, 2)                     # [H, R, D]
    ks = kf[None].expand(qs.shape[0], -1, -1)
    vs = vf[None].expand(qs.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(
        qs, ks, vs, attn_mask=mask[None], scale=scale)  # [H, R, Dv]
    logits = (qs @ kf.T) * scale                       # [H, R, S_k]
    logits = logits.masked_fill(~mask[None], float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)              # [H, R]
    return o.permute(1, 0, 2).numpy(), lse.T.numpy()
