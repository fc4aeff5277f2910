"""Seeded synthetic inputs for the DSA forward path.

This module only draws random numbers and casts them to the storage types;
it holds none of the method's arithmetic, so both the GPU path and the CPU
oracle can consume its arrays.

The workloads follow the shapes the SkyRL blog "Scaling Training to 1M Token
Context on GLM-5.3-Flash" describes for the DSA layers of GLM-5.3-Flash (section
"DeepSeek Sparse Attention (DSA) Optimizations": pools of 4 tokens, 2048
selected tokens; "Making Sparse Attention Actually Sparse": NoPE heads and
2,051 keys; "Over Time: Chunking": a few hundred queries per chunk; "Across
GPUs: Sharding": one GPU's share of the queries).  The page's throughput
and memory figures come from synthetic runs (untrained weights, random token
ids; section "Intro"), so seeded random inputs match its own workload.

Recipe: numpy PCG64 seeded with ``seed`` (by default 1000 + the workload
number), seven independent sub-streams from ``SeedSequence(seed).spawn(7)``
in the fixed order [q_idx, k_idx, w, q, k, v, knorm]; values drawn in fp32
and cast to bf16 (round to nearest even) or to fp8 E4M3 by torch.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    number: int            # 1-based position in the workload list
    s_q: int               # queries
    s_k: int               # keys / values
    q_pos0: int            # position of the first query in the sequence
    h_idx: int             # indexer heads
    d_idx: int             # indexer head dim
    k_pools: int           # pools selected per query
    h: int                 # attention query heads (one shared KV head)
    d: int                 # attention head dim (q, k)
    dv: int                # value head dim
    n_tail: int            # own-pool tokens attended besides the selected pools
    idx_std: float         # std of q_idx, k_idx
    attn_std: float        # std of q, k, v
    knorm_sigma: float     # log-normal row scale of the indexer keys (0 = none)
    chunk_q: int           # queries scored and selected per chunk
    fp8: bool = False      # also run the fp8 E4M3 indexer variant

    @property
    def seed(self) -> int:
        return 1000 + self.number

    @property
    def n_pools(self) -> int:
        return self.s_k // 4


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_s2048", 1, 2048, 2048, 0, 4, 64, 128, 8, 64, 64, 0,
                 1.0 / 8, 1.0, 0.0, 256),
        Workload("s32k", 2, 32768, 32768, 0, 32, 128, 512, 16, 128, 128, 0,
                 1.0 / math.sqrt(128), 1.0 / math.sqrt(128), 0.0, 256),
        Workload("s128k", 3, 131072, 131072, 0, 32, 128, 512, 16, 128, 128, 0,
                 1.0 / math.sqrt(128), 1.0 / math.sqrt(128), 0.5, 256),
        Workload("nope_s64k", 4, 65536, 65536, 0, 32, 96, 512, 16, 96, 96, 3,
                 1.0, 1.0, 0.0, 256, fp8=True),
        Workload("share_1m", 5, 131072, 1048576, 917504, 32, 128, 512, 16, 128, 128, 0,
                 1.0, 1.0, 0.0, 256),
    ]
}
WORKLOAD_LIST = sorted(WORKLOADS.values(), key=lambda w: w.number)


def custom(name: str = "custom", *, s_q: int, s_k: int | None = None, q_pos0: int = 0,
           h_idx: int = 32, d_idx: int = 128, k_pools: int = 512, h: int = 16, d: int = 128,
           dv: int | None = None, n_tail: int = 0, idx_std: float = 1.0,
           attn_std: float = 1.0, knorm_sigma: float = 0.0, chunk_q: int = 256,
           fp8: bool = False, number: int = 100) -> Workload:
    """A workload of any shape with the same distributions (for tests)."""
    return Workload(name, number, s_q, s_k if s_k is not None else q_pos0 + s_q, q_pos0, h_idx,
                    d_idx, k_pools, h, d, dv if dv is not None else d, n_tail, idx_std,
                    attn_std, knorm_sigma, chunk_q, fp8)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def make_inputs(wl: Workload, seed: int | None = None, *, attention: bool = True,
                indexer: bool = True, w_per_query: bool = False) -> dict:
    """Host (CPU) tensors for one workload.

    Returns a dict with q_idx [S_q,H_I,D_I] bf16, k_idx [S_k,D_I] bf16,
    w [H_I] fp32 (one row for every query; [S_q,H_I] when ``w_per_query``),
    q [S_q,H,D], k [S_k,D], v [S_k,Dv] bf16, and, for fp8 workloads,
    q_idx8 / k_idx8 (E4M3 codes of the same draws, per-tensor scale 1).
    """
    seed = wl.seed if seed is None else seed
    ss = np.random.SeedSequence(seed).spawn(7)
    g = [np.random.Generator(np.random.PCG64(s)) for s in ss]
    out: dict = {}
    if indexer:
        qi = _normal(g[0], (wl.s_q, wl.h_idx, wl.d_idx), wl.idx_std)
        ki = _normal(g[1], (wl.s_k, wl.d_idx), wl.idx_std)
        if wl.knorm_sigma > 0:
            # log-normal row scale, drawn from its own sub-stream
            scale = np.exp(np.float32(wl.knorm_sigma) *
                           g[6].standard_normal(size=(wl.s_k, 1), dtype=np.float32))
            ki *= scale.astype(np.float32)
        if w_per_query:
            w = g[2].random(size=(wl.s_q, wl.h_idx), dtype=np.float32)
        else:
            w = g[2].random(size=(wl.h_idx,), dtype=np.float32)
        out["q_idx"] = torch.from_numpy(qi).to(torch.bfloat16)
        out["k_idx"] = torch.from_numpy(ki).to(torch.bfloat16)
        if wl.fp8:
            out["q_idx8"] = torch.from_numpy(qi).to(torch.float8_e4m3fn)
            out["k_idx8"] = torch.from_numpy(ki).to(torch.float8_e4m3fn)
        del qi, ki
        out["w"] = torch.from_numpy(w)
    if attention:
        out["q"] = torch.from_numpy(_normal(g[3], (wl.s_q, wl.h, wl.d), wl.attn_std)).to(torch.bfloat16)
        out["k"] = torch.from_numpy(_normal(g[4], (wl.s_k, wl.d), wl.attn_std)).to(torch.bfloat16)
        out["v"] = torch.from_numpy(_normal(g[5], (wl.s_k, wl.dv), wl.attn_std)).to(torch.bfloat16)
    return out


def make_gates(wl: Workload, seed: int | None = None) -> torch.Tensor:
    """Per-token k-pool gate scores [S_k] fp32 for gated pooling.

    Drawn U(0, 1) from an eighth sub-stream of the same seed (the first seven
    are those of ``make_inputs``), then normalised so that the 4 gates of each
    pool sum to 1: the caller supplies normalised gates.  Keys past the last
    whole pool get gate 0."""
    seed = wl.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(8)[7]))
    u = rng.random(size=(wl.s_k,), dtype=np.float32) + np.float32(1e-3)
    g = np.zeros_like(u)
    n = wl.n_pools * 4
    pools = u[:n].reshape(-1, 4)
    g[:n] = (pools / pools.sum(axis=1, keepdims=True, dtype=np.float32)).reshape(-1)
    return torch.from_numpy(g)


def make_dout(wl: Workload, seed: int | None = None) -> torch.Tensor:
    """Upstream gradient of the attention output, dout [S_q, H, Dv] bf16,
    N(0, 1) from a ninth sub-stream of the same seed (the first eight are
    those of ``make_inputs`` and ``make_gates``)."""
    seed = wl.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(9)[8]))
    return torch.from_numpy(_normal(rng, (wl.s_q, wl.h, wl.dv), 1.0)).to(torch.bfloat16)


def sample_rows(s_q: int, n: int, extra=()) -> np.ndarray:
    """Rows for sampled checks: the first and last rows, rows around every
    4-aligned boundary near the ends, a strided sweep, plus ``extra``."""
    if n >= s_q:
        return np.arange(s_q, dtype=np.int64)
    base = list(range(min(8, s_q))) + list(range(max(0, s_q - 8), s_q))
    stride = max(1, s_q // max(1, n - len(base)))
    base += list(range(stride // 2, s_q, stride))
    base += [r for r in extra if 0 <= r < s_q]
    return np.array(sorted(set(base)), dtype=np.int64)
