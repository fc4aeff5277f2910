"""Parity rules between the GPU path and the CPU oracle.

Index sets (pages: SkyRL blog, section "DeepSeek Sparse Attention (DSA)
Optimizations" -- keep the best pools; the sets must be exact except where
pools tie at the k-th score to within rounding, read as the band below):
  * rows with n(t) <= k must equal [0 .. n(t)-1] padded with -1, exactly;
  * other rows must hold k distinct, ascending, eligible ids, and the
    symmetric difference with the oracle's set may only contain pools whose
    oracle fp32 score lies in the boundary band
        |s(p) - s_k| <= 1e-3 |s_k| + 1e-6 max_p s(p)
    around the oracle's k-th score s_k (counted and reported).
Scores: |s_gpu - s_ref| <= 1e-2 |s_ref| + 1e-4 max_p |s_ref(t, p)| per row.
Attention (oracle fed the GPU's ids): |o_gpu - o_ref| <= 2e-2 and
|lse_gpu - lse_ref| <= 2e-2, absolute, for bf16 inputs/outputs with fp32
accumulation on the GPU.
Attention backward (no tolerance is given by the pages; this one follows
from the arithmetic): every gradient element is a sum of terms
c_a * x_a (dS_a k_a, dS_a q, P_a dout), and the GPU rounds P_a and dS_a to
bf16 for the matrix cores (relative 2^-9) and takes D from the stored bf16
forward output, whose error is at most 2^-8 sum_a P_a |v_a| per element, so
|dD| <= 2^-8 Dabs.  Each term's error is then at most 2^-8 m_a |x_a| with
m_a = |dS_a| + P_a Dabs (the oracle's magnitude sums), and fp32 summation
over the chains the kernels use (at most a few thousand partial sums) adds
far less than another 2^-8.  The bound is
    |g_gpu - g_ref| <= 2^-6 * mag   elementwise,  and g_gpu == 0 where mag == 0.
"""
from __future__ import annotations

import numpy as np

BAND_REL = 1e-3
BAND_ABS_OF_MAX = 1e-6
SCORE_REL = 1e-2
SCORE_ABS_OF_MAX = 1e-4
ATTN_ABS = 2e-2


def eligible(t: int, n_pools: int) -> int:
    return min(t // 4, n_pools)


def validate_index_rows(idx: np.ndarray, positions, n_pools: int, k: int) -> None:
    """Host-side structural check of id rows before they feed attention,
    which trusts them: a row for position t holds m = min(n(t), k) distinct
    pool ids in strictly ascending order, each with 4p + 3 < t (p < n(t)),
    followed by k - m entries of -1.  Vectorised, so it runs on every row of
    a full-size output."""
    idx = np.asarray(idx)
    pos = np.asarray(positions, dtype=np.int64)
    assert idx.ndim == 2 and idx.shape == (len(pos), k), f"id rows of shape {idx.shape}"
    n = np.minimum(pos // 4, n_pools)
    m = np.minimum(n, k)
    valid = np.arange(k)[None, :] < m[:, None]
    bad_pad = (~valid) & (idx != -1)
    assert not bad_pad.any(), f"rows {np.nonzero(bad_pad.any(1))[0][:8]}: padding is not -1"
    bad_rng = valid & ((idx < 0) | (idx >= n[:, None]))
    assert not bad_rng.any(), \
        f"rows {np.nonzero(bad_rng.any(1))[0][:8]}: id not strictly before the query's pool"
    both = valid[:, 1:] & valid[:, :-1]
    bad_ord = both & (idx[:, 1:] <= idx[:, :-1])
    assert not bad_ord.any(), f"rows {np.nonzero(bad_ord.any(1))[0][:8]}: ids not ascending"


# (case label, stats) of every index comparison made in this process; the
# test session writes them out when DSA_PARITY_RECORD names a file
SWAP_LOG: list = []


def check_index_rows(gpu_idx: np.ndarray, ora_idx: np.ndarray, ora_scores: np.ndarray,
                     positions, n_pools: int, k: int, label: str | None = None) -> dict:
    """gpu_idx / ora_idx [R, k] int32; ora_scores [R, P] fp32 (dense oracle
    scores of the same rows); positions [R] sequence positions t.  Returns
    the boundary-swap counts (and logs them under ``label``)."""
    swaps = 0
    rows_with_swaps = 0
    worst = 0
    nontrivial = 0
    validate_index_rows(gpu_idx, positions, n_pools, k)
    for r, t in enumerate(positions):
        n = eligible(int(t), n_pools)
        g = gpu_idx[r]
        o = ora_idx[r]
        if n <= k:
            expect = np.concatenate([np.arange(n), -np.ones(k - n)]).astype(np.int32)
            assert np.array_equal(g, expect), f"row t={t}: trivial row differs"
            assert np.array_equal(o, expect), f"row t={t}: oracle trivial row differs"
            continue
        nontrivial += 1
        assert np.all(g >= 0) and np.all(g < n), f"row t={t}: id out of range"
        assert np.all(np.diff(g) > 0), f"row t={t}: ids not strictly ascending"
        gs, os_ = set(g.tolist()), set(o.tolist())
        diff = gs ^ os_
        if diff:
            s = ora_scores[r, :n]
            # oracle k-th score in its own order (descending score, ascending id)
            s_k = s[o].min()
            band = BAND_REL * abs(s_k) + BAND_ABS_OF_MAX * s.max()
            bad = [p for p in diff if abs(float(s[p]) - float(s_k)) > band]
            assert not bad, (f"row t={t}: pools {bad[:8]} differ outside the boundary band "
                             f"(s_k={s_k}, scores {[float(s[p]) for p in bad[:8]]})")
            sw = len(gs - os_)
            swaps += sw
            rows_with_swaps += 1
            worst = max(worst, sw)
    stats = {"swaps": swaps, "rows_with_swaps": rows_with_swaps, "worst_row": worst,
             "rows": len(positions), "rows_beyond_k": nontrivial}
    if label is not None:
        SWAP_LOG.append((label, stats))
    return stats


def write_swap_record(path: str) -> None:
    """Markdown table of the logged index comparisons."""
    lines = ["| case | rows checked | rows with n(t) > k | swaps | rows with swaps | "
             "largest swaps in a row |", "|---|---|---|---|---|---|"]
    tot = {"rows": 0, "rows_beyond_k": 0, "swaps": 0, "rows_with_swaps": 0, "worst_row": 0}
    for label, st in SWAP_LOG:
        lines.append(f"| {label} | {st['rows']} | {st['rows_beyond_k']} | {st['swaps']} | "
                     f"{st['rows_with_swaps']} | {st['worst_row']} |")
        for key in tot:
            tot[key] = max(tot[key], st[key]) if key == "worst_row" else tot[key] + st[key]
    lines.append(f"| **all** | {tot['rows']} | {tot['rows_beyond_k']} | {tot['swaps']} | "
                 f"{tot['rows_with_swaps']} | {tot['worst_row']} |")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def check_scores(gpu: np.ndarray, ref: np.ndarray) -> float:
    """Dense rows [R, P]; -inf entries must coincide.  Returns the worst
    error relative to the allowed bound."""
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(gpu)), "eligibility pattern differs"
    worst = 0.0
    for r in range(ref.shape[0]):
        f = fin[r]
        if not f.any():
            continue
        rr = ref[r, f].astype(np.float64)
        gg = gpu[r, f].astype(np.float64)
        bound = SCORE_REL * np.abs(rr) + SCORE_ABS_OF_MAX * np.abs(rr).max()
        err = np.abs(gg - rr)
        ratio = (err / np.maximum(bound, 1e-30)).max()
        assert np.all(err <= bound), f"row {r}: score error {err.max()} beyond bound"
        worst = max(worst, float(ratio))
    return worst


def check_attention(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray,
                    lse_ref: np.ndarray) -> tuple[float, float]:
    err_o = np.abs(o_gpu.astype(np.float64) - o_ref)
    assert err_o.max() <= ATTN_ABS, f"attention output error {err_o.max()}"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(empty, np.isneginf(lse_gpu)), "empty-row pattern differs"
    err_l = np.abs(lse_gpu[~empty].astype(np.float64) - lse_ref[~empty]) if (~empty).any() \
        else np.zeros(1)
    assert err_l.max() <= ATTN_ABS, f"lse error {err_l.max()}"
    return float(err_o.max()), float(err_l.max())


BWD_MAG_REL = 2.0 ** -6


def check_grad(name: str, gpu: np.ndarray, ref: np.ndarray, mag: np.ndarray) -> float:
    """Returns the worst error relative to the bound (<= 1 passes)."""
    g = gpu.astype(np.float64)
    err = np.abs(g - ref)
    zero = mag == 0
    assert np.all(g[zero] == 0), f"{name}: nonzero where no term contributes"
    bound = BWD_MAG_REL * mag
    ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, bound))
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{name}: error {err[i]:.3g} at {i} beyond the bound {bound[i]:.3g} "
                             f"(gpu {g[i]:.6g}, ref {ref[i]:.6g})")
    return worst
