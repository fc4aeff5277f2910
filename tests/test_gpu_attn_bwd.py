"""GPU parity of the sparse-attention backward (dq, dk, dv) through the C ABI
against the fp64 CPU oracle.

The pages' setting is training (SkyRL blog, section "Activation Recompute":
the forward is rerun inside the backward pass); the backward recomputes the
softmax weights from the forward's lse.  The kept-pool rows are drawn on the
host (seeded, one id from each of k equal strata of the eligible pools), the
GPU forward supplies out and lse to the GPU backward, and the oracle works
from the same q, k, v, idx and dout alone.  Full-size workloads zero dout
outside a sample of rows: dk and dv then hold exactly the sampled rows'
contributions, which the oracle computes one row at a time.  Bound:
tests/parity.py (2^-6 of the oracle's magnitude sums, exact zeros where no
term contributes).
"""
import math

import numpy as np
import pytest
import torch

from long_context_sparse_dsa_amd import dsa, inputs
from oracle import oracle
import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.load_library()


def stratified_idx(s_q, q_pos0, n_pools, k, seed, block=16384):
    """Kept-pool rows [s_q, k] int32: every eligible pool (then -1) when a
    query has at most k, else one id drawn from each of k equal strata of
    [0, n(t)) -- distinct and ascending by construction."""
    rng = np.random.default_rng(seed)
    out = np.empty((s_q, k), dtype=np.int32)
    j = np.arange(k, dtype=np.int64)[None, :]
    for r0 in range(0, s_q, block):
        r1 = min(s_q, r0 + block)
        t = q_pos0 + np.arange(r0, r1, dtype=np.int64)
        n = np.minimum(t // 4, n_pools)[:, None]
        lo = (n * j) // k
        hi = (n * (j + 1)) // k
        pick = lo + np.floor(rng.random((r1 - r0, k)) * (hi - lo)).astype(np.int64)
        ids = np.where(n <= k, j, pick)
        out[r0:r1] = np.where(j < np.minimum(n, k), ids, -1)
    return out


def skewed_idx(s_q, q_pos0, n_pools, k, seed, sigma=2.0):
    """Kept-pool rows [s_q, k] int32 where a few pools are kept by most
    queries: each query draws k distinct eligible pools with probability
    proportional to a per-pool log-normal weight (sigma), sorted ascending;
    every eligible pool (then -1) when a query has at most k."""
    rng = np.random.default_rng(seed)
    weight = np.exp(sigma * rng.standard_normal(n_pools))
    out = np.full((s_q, k), -1, dtype=np.int32)
    for r in range(s_q):
        n = min((q_pos0 + r) // 4, n_pools)
        if n <= k:
            out[r, :n] = np.arange(n)
            continue
        p = weight[:n] / weight[:n].sum()
        out[r] = np.sort(rng.choice(n, size=k, replace=False, p=p))
    return out


def run_bwd(wl, rows=None, chunk_q=0, seed=None, idx=None, check=True):
    seed = wl.seed if seed is None else seed
    _say(f"[bwd] {wl.name} s_q={wl.s_q} s_k={wl.s_k} q_pos0={wl.q_pos0} H={wl.h} D={wl.d} "
         f"Dv={wl.dv} k={wl.k_pools} n_tail={wl.n_tail} chunk_q={chunk_q} seed={seed} "
         f"rows={'all' if rows is None else len(rows)}")
    x = inputs.make_inputs(wl, seed=seed, indexer=False)
    dout = inputs.make_dout(wl, seed=seed)
    if idx is None:
        idx = stratified_idx(wl.s_q, wl.q_pos0, wl.n_pools, wl.k_pools, seed)
    if rows is None:
        rows = np.arange(wl.s_q)
    else:
        keep = torch.zeros(wl.s_q, dtype=torch.bool)
        keep[torch.from_numpy(np.asarray(rows))] = True
        dout = torch.where(keep[:, None, None], dout, torch.zeros_like(dout))
    dev = torch.device("cuda")
    q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
    idx_d = torch.from_numpy(idx).to(dev)
    o, lse = dsa.dsa_sparse_attn_fwd(q, k, v, idx_d, q_pos0=wl.q_pos0, n_tail=wl.n_tail,
                                     want_lse=True)
    dq, dk, dv = dsa.dsa_sparse_attn_bwd(q, k, v, idx_d, o, dout.to(dev), lse, q_pos0=wl.q_pos0,
                                         n_tail=wl.n_tail, chunk_q=chunk_q)
    torch.cuda.synchronize()
    got = {"dq": dq.cpu().numpy(), "dk": dk.cpu().numpy(), "dv": dv.cpu().numpy()}
    if not check:
        return got
    scale = float(np.float32(1.0 / math.sqrt(wl.d)))
    ref = oracle.sparse_attn_bwd(x["q"], x["k"], x["v"], idx[rows], dout, wl.k_pools,
                                 q_pos0=wl.q_pos0, rows=rows, n_tail=wl.n_tail, scale=scale,
                                 magnitudes=True)
    w = {"dq": parity.check_grad("dq", got["dq"][rows], ref["dq"], ref["dq_mag"]),
         "dk": parity.check_grad("dk", got["dk"], ref["dk"], ref["dk_mag"]),
         "dv": parity.check_grad("dv", got["dv"], ref["dv"], ref["dv_mag"])}
    if len(rows) < wl.s_q:
        others = np.setdiff1d(np.arange(wl.s_q), rows)
        assert np.all(got["dq"][others] == 0), "dq of a row with zero dout is not zero"
    _say("  worst error / bound: " + ", ".join(f"{n} {r:.3g}" for n, r in w.items()))
    return got


SMALL = [
    # s_q, s_k, q_pos0, h, d, dv, k_pools, n_tail, chunk_q
    (300, 300, 0, 4, 64, 64, 8, 0, 0),
    (517, 517, 0, 16, 128, 128, 16, 3, 64),
    (450, 450, 0, 16, 96, 96, 12, 3, 128),
    (200, 203, 0, 1, 64, 128, 5, 2, 64),       # one head, s_k with a partial pool
    (333, 1000, 667, 5, 128, 96, 40, 1, 64),   # queries late in the sequence
    (129, 131, 2, 16, 128, 64, 64, 3, 0),      # k covers every pool: dense causal
    (2500, 2500, 0, 2, 64, 64, 4, 1, 2560),    # 80 bitmap words per chunk: two scan windows
    (3000, 3001, 0, 16, 96, 96, 6, 3, 2048),   # two chunks (2048 and 952 queries)
    # 282 bitmap words in one chunk (five scan windows of 64 words); the first
    # pools are kept by nearly every query, so the first pool groups walk
    # thousands of entries
    (9000, 9000, 0, 2, 64, 64, 512, 1, 9024),
    (2600, 2600, 0, 4, 128, 128, 200, 3, 0),   # about 1700 entries in the first groups
    (3000, 3000, 0, 4, 64, 64, 700, 1, 0),     # rows of more than 512 ids (a second id pass)
]


@pytest.mark.parametrize("s_q,s_k,q_pos0,h,d,dv,k_pools,n_tail,chunk_q", SMALL)
def test_small_all_rows(s_q, s_k, q_pos0, h, d, dv, k_pools, n_tail, chunk_q):
    wl = inputs.custom("bwd_small", s_q=s_q, s_k=s_k, q_pos0=q_pos0, h=h, d=d, dv=dv,
                       k_pools=k_pools, n_tail=n_tail)
    run_bwd(wl, chunk_q=chunk_q, seed=s_q + h)


@pytest.mark.parametrize("chunk_q", [0, 256])
def test_popular_pools_all_rows(chunk_q):
    # the key-major pass groups the pool slots by how many queries of the
    # last chunk keep them: with skewed selections its groups hold slots from
    # all over the sequence (also the query's own pool, whose tail tokens are
    # attended, and the padding slots of 2003 keys = 500 pools and 3 tokens,
    # 501 slots)
    wl = inputs.custom("bwd_popular", s_q=2000, s_k=2003, h=16, d=128, dv=128, k_pools=48,
                       n_tail=3)
    idx = skewed_idx(wl.s_q, wl.q_pos0, wl.n_pools, wl.k_pools, seed=77)
    kept = np.bincount(idx[idx >= 0], minlength=wl.n_pools)
    assert kept.max() > wl.s_q // 2, "the draw should make some pools popular"
    run_bwd(wl, chunk_q=chunk_q, seed=78, idx=idx)


def test_deterministic_bitwise():
    wl = inputs.custom("bwd_det", s_q=700, s_k=700, h=16, d=128, k_pools=24, n_tail=3)
    a = run_bwd(wl, chunk_q=128, seed=3, check=False)
    b = run_bwd(wl, chunk_q=128, seed=3, check=False)
    for n in a:
        assert np.array_equal(a[n].view(np.uint32), b[n].view(np.uint32)), n


def test_chunking_leaves_dq_bitwise_and_dkdv_in_bound():
    wl = inputs.custom("bwd_chunks", s_q=640, s_k=640, h=8, d=64, k_pools=20, n_tail=2)
    one = run_bwd(wl, chunk_q=0, seed=4)
    many = run_bwd(wl, chunk_q=64, seed=4)
    assert np.array_equal(one["dq"], many["dq"])


def test_rows_without_tokens_and_empty_queries():
    # every kept id invalid and no tail: the rows see nothing, dq = 0, dk = dv = 0
    wl = inputs.custom("bwd_empty", s_q=64, s_k=64, h=4, d=64, k_pools=4, n_tail=0)
    idx = np.full((64, 4), -1, dtype=np.int32)
    got = run_bwd(wl, idx=idx, seed=5)
    assert np.all(got["dq"] == 0) and np.all(got["dk"] == 0) and np.all(got["dv"] == 0)
    # no query at all: the key and value gradients are zero
    dev = torch.device("cuda")
    k = torch.randn(40, 64, device=dev).bfloat16()
    v = torch.randn(40, 64, device=dev).bfloat16()
    q = torch.empty((0, 4, 64), device=dev, dtype=torch.bfloat16)
    o = torch.empty((0, 4, 64), device=dev, dtype=torch.bfloat16)
    lse = torch.empty((0, 4), device=dev)
    ix = torch.empty((0, 4), device=dev, dtype=torch.int32)
    dk = torch.full((40, 64), 7.0, device=dev)
    dv = torch.full((40, 64), 7.0, device=dev)
    dsa.dsa_sparse_attn_bwd(q, k, v, ix, o, o, lse, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


# ------------------------------------------------------------ full-size workloads
# The benchmark's launch configuration (default chunk); dout is zero outside
# the sampled rows, so dk and dv carry exactly their contributions.

def _sampled(name, n):
    wl = inputs.WORKLOADS[name]
    rows = inputs.sample_rows(wl.s_q, n)
    run_bwd(wl, rows=rows)


@pytest.mark.slow
def test_workload_s32k_sampled():
    _sampled("s32k", 256)


@pytest.mark.slow
def test_workload_s128k_sampled():
    _sampled("s128k", 512)


@pytest.mark.slow
def test_workload_nope_s64k_sampled():
    _sampled("nope_s64k", 256)


@pytest.mark.slow
def test_workload_share_1m_sampled():
    _sampled("share_1m", 256)


@pytest.mark.slow
def test_per_chunk_bitmaps_with_a_short_last_chunk():
    # 1M keys and 33000 queries: the bitmaps of all chunks would exceed 1 GiB,
    # so each chunk's is built in turn (8192-query chunks, the last of 232),
    # and the pool groups are ordered from the last 8192 queries, which span
    # two chunks
    wl = inputs.custom("bwd_per_chunk", s_q=33000, s_k=1 << 20, q_pos0=(1 << 20) - 33000,
                       h=16, d=128, dv=128, k_pools=512, n_tail=0)
    nbytes, cq = dsa.dsa_sparse_attn_bwd_workspace_size(wl.s_q, wl.s_k, wl.h)
    assert cq == 8192 and nbytes < (1 << 30)
    ends = [r for c0 in range(0, wl.s_q, cq) for r in (c0, min(wl.s_q, c0 + cq) - 1)]
    run_bwd(wl, rows=inputs.sample_rows(wl.s_q, 64, extra=ends))


@pytest.mark.slow
def test_workload_s128k_indexer_ids_sampled():
    # the backward as the benchmark runs it: ids from the indexer on the
    # workload's own keys (pools with large key norms are kept by many
    # queries, so some pool groups walk far more entries than the rest)
    wl = inputs.WORKLOADS["s128k"]
    _say(f"[bwd] {wl.name}: ids from dsa_index_score_topk (k={wl.k_pools})")
    x = inputs.make_inputs(wl, attention=False)
    dev = torch.device("cuda")
    idx, _ = dsa.dsa_index_score_topk(x["q_idx"].to(dev), x["k_idx"].to(dev), x["w"].to(dev),
                                      wl.k_pools, q_pos0=wl.q_pos0)
    idx = idx.cpu().numpy()
    del x
    run_bwd(wl, rows=inputs.sample_rows(wl.s_q, 256), idx=idx)
