"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case prints what it runs before touching the GPU.  Each case runs the
indexer twice: with the kept scores requested (score_out) and without them,
the call the benchmark times.  The two id arrays must be identical bit for
bit, every id row must pass the host-side structural check (causal,
ascending, -1 padded) before it feeds attention, and the ids are compared
with the oracle's under the boundary rule.  Small cases check every row; the
full-size workloads check sampled rows (first and last rows, 4-aligned
boundaries, a strided sweep, the first and last row of every chunk) with the
default chunking, as the benchmark runs it.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

from long_context_sparse_dsa_amd import dsa, inputs
from oracle import oracle
import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.load_library()


def run_case(wl, rows=None, chunk_q=0, w_per_query=False, attention=True, seed=None,
             check_scores=True, x=None, fp8=False, scales=(1.0, 1.0), gate=None, tag=""):
    _say(f"[case] {wl.name} s_q={wl.s_q} s_k={wl.s_k} q_pos0={wl.q_pos0} "
         f"H_I={wl.h_idx} D_I={wl.d_idx} k={wl.k_pools} H={wl.h} D={wl.d} Dv={wl.dv} "
         f"n_tail={wl.n_tail} chunk_q={chunk_q} fp8={fp8} scales={scales} "
         f"gated={gate is not None} seed={seed if seed is not None else wl.seed}")
    if x is None:
        x = inputs.make_inputs(wl, seed=seed, attention=attention, w_per_query=w_per_query)
    dev = torch.device("cuda")
    qn, kn = ("q_idx8", "k_idx8") if fp8 else ("q_idx", "k_idx")
    q_idx, k_idx, w = (x[qn].to(dev), x[kn].to(dev), x["w"].to(dev))
    sc_kw = {}
    if fp8:
        sc_kw = dict(q_scale=torch.tensor([scales[0]], dtype=torch.float32, device=dev),
                     k_scale=torch.tensor([scales[1]], dtype=torch.float32, device=dev))
    g_dev = None if gate is None else gate.to(dev)
    g_np = None if gate is None else gate.numpy()

    def indexer(want_scores):
        if gate is None:
            return dsa.dsa_index_score_topk(q_idx, k_idx, w, wl.k_pools, q_pos0=wl.q_pos0,
                                            chunk_q=chunk_q, want_scores=want_scores, **sc_kw)
        return dsa.dsa_index_score_topk_gated(q_idx, k_idx, g_dev, w, wl.k_pools,
                                              q_pos0=wl.q_pos0, chunk_q=chunk_q,
                                              want_scores=want_scores, **sc_kw)

    idx_g, sc_g = indexer(True)
    # the benchmark's call: no score_out (other branches in the chunk loop
    # and the selection), same ids required
    idx_b, _ = indexer(False)
    torch.cuda.synchronize()
    assert torch.equal(idx_g, idx_b), "ids without score_out differ from ids with it"
    idx_all = idx_b.cpu().numpy()
    parity.validate_index_rows(idx_all, wl.q_pos0 + np.arange(wl.s_q), wl.n_pools, wl.k_pools)
    rows = np.arange(wl.s_q) if rows is None else np.asarray(rows, dtype=np.int64)
    pos = wl.q_pos0 + rows
    idx_g_rows = idx_all[rows]
    sc_g_rows = sc_g.cpu().numpy()[rows]
    def oracle_rows(rs):
        if fp8:
            i_o, c_o = oracle.index_topk_fp8(x[qn], x[kn], x["w"], wl.k_pools, q_scale=scales[0],
                                             k_scale=scales[1], q_pos0=wl.q_pos0, rows=rs,
                                             gate=g_np)
            d_o = oracle.index_scores_fp8(x[qn], x[kn], x["w"], q_scale=scales[0],
                                          k_scale=scales[1], q_pos0=wl.q_pos0, rows=rs, gate=g_np)
        else:
            i_o, c_o = oracle.index_topk(x["q_idx"], x["k_idx"], x["w"], wl.k_pools,
                                         q_pos0=wl.q_pos0, rows=rs, gate=g_np)
            d_o = oracle.index_scores(x["q_idx"], x["k_idx"], x["w"], q_pos0=wl.q_pos0, rows=rs,
                                      gate=g_np)
        return i_o, c_o, d_o

    # long row lists go to the oracle in batches, each reported when done
    batch = 256 if len(rows) > 512 else len(rows)
    parts = []
    for b0 in range(0, len(rows), max(1, batch)):
        parts.append(oracle_rows(rows[b0:b0 + batch]))
        if batch < len(rows):
            _say(f"  oracle rows {min(len(rows), b0 + batch)}/{len(rows)}")
    if parts:
        idx_o, sc_o, s_o = (np.concatenate([p[j] for p in parts]) for j in range(3))
    else:
        idx_o, sc_o, s_o = oracle_rows(rows)
    label = (f"{wl.name} (s_q={wl.s_q}, s_k={wl.s_k}, k={wl.k_pools}, chunk_q={chunk_q or 'default'}"
             f"{', fp8' if fp8 else ''}{', gated' if gate is not None else ''}"
             f"{', ' + tag if tag else ''})")
    stats = parity.check_index_rows(idx_g_rows, idx_o, s_o, pos, wl.n_pools, wl.k_pools,
                                    label=label)
    _say(f"  index: {stats}")
    # the kept pools' scores against the oracle's dense scores
    for r in range(len(rows)):
        sel = idx_g_rows[r] >= 0
        ref = s_o[r][idx_g_rows[r][sel]]
        got = sc_g_rows[r][sel]
        if sel.any():
            bound = parity.SCORE_REL * np.abs(ref) + parity.SCORE_ABS_OF_MAX * np.abs(
                s_o[r][np.isfinite(s_o[r])]).max()
            assert np.all(np.abs(got - ref) <= bound), f"row {rows[r]}: kept-pool scores differ"
        assert np.all(np.isneginf(sc_g_rows[r][~sel]))
    if check_scores:
        # dense scores of a few contiguous row blocks
        blocks = sorted(set([0, max(0, wl.s_q // 2 - 8), max(0, wl.s_q - 16)]))
        worst = 0.0
        for b0 in blocks:
            nb = min(16, wl.s_q - b0)
            if gate is None:
                g = dsa.dsa_index_scores(q_idx, k_idx, w, row0=b0, n_rows=nb, q_pos0=wl.q_pos0,
                                         **sc_kw)
            else:
                g = dsa.dsa_index_scores_gated(q_idx, k_idx, g_dev, w, row0=b0, n_rows=nb,
                                               q_pos0=wl.q_pos0, **sc_kw)
            if fp8:
                ref = oracle.index_scores_fp8(x[qn], x[kn], x["w"], q_scale=scales[0],
                                              k_scale=scales[1], q_pos0=wl.q_pos0,
                                              rows=np.arange(b0, b0 + nb), gate=g_np)
            else:
                ref = oracle.index_scores(x["q_idx"], x["k_idx"], x["w"], q_pos0=wl.q_pos0,
                                          rows=np.arange(b0, b0 + nb), gate=g_np)
            worst = max(worst, parity.check_scores(g.cpu().numpy(), ref))
        _say(f"  scores: worst error / bound = {worst:.3g}")
    if attention:
        q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
        o_g, lse_g = dsa.dsa_sparse_attn_fwd(q, k, v, idx_b, q_pos0=wl.q_pos0,
                                             n_tail=wl.n_tail, want_lse=True)
        torch.cuda.synchronize()
        scale = float(np.float32(1.0 / math.sqrt(wl.d)))
        o_o, lse_o = oracle.sparse_attn(x["q"], x["k"], x["v"], idx_g_rows, wl.k_pools,
                                        q_pos0=wl.q_pos0, rows=rows, n_tail=wl.n_tail,
                                        scale=scale)
        eo, el = parity.check_attention(o_g.float().cpu().numpy()[rows],
                                        lse_g.cpu().numpy()[rows], o_o, lse_o)
        _say(f"  attention: max |do| = {eo:.3g}, max |dlse| = {el:.3g}")
    return x, idx_b


# ---------------------------------------------------------------- gated pooling
# section "DSA: Gather by Token Position": per-token k-pool gate scores weight
# each key within its pool.

@pytest.mark.parametrize("h_idx,d_idx,fp8", [(32, 128, False), (16, 96, False), (4, 64, False),
                                             (32, 96, True), (8, 128, True)])
def test_gated_pooling(h_idx, d_idx, fp8):
    # k small against the rows' lengths: most chunks take the bounded path
    wl = inputs.custom(f"gated_{h_idx}x{d_idx}{'_fp8' if fp8 else ''}", s_q=1300, s_k=1303,
                       h_idx=h_idx, d_idx=d_idx, k_pools=8, h=16, d=d_idx,
                       idx_std=1.0 if fp8 else 1 / math.sqrt(d_idx),
                       attn_std=1 / math.sqrt(d_idx), fp8=fp8, number=400 + h_idx + d_idx)
    gate = inputs.make_gates(wl)
    run_case(wl, chunk_q=192, w_per_query=True, fp8=fp8, gate=gate,
             attention=not fp8)


@pytest.mark.parametrize("fp8", [False, True])
def test_quarter_gates_reproduce_mean_pooling_bitwise(fp8):
    wl = inputs.custom("quarter_gates", s_q=900, s_k=900, h_idx=16, d_idx=128, k_pools=40,
                       idx_std=1.0 if fp8 else 0.1, fp8=fp8, number=420)
    _say(f"[case] quarter gates fp8={fp8}")
    x = inputs.make_inputs(wl, attention=False)
    dev = torch.device("cuda")
    qn, kn = ("q_idx8", "k_idx8") if fp8 else ("q_idx", "k_idx")
    q_idx, k_idx, w = x[qn].to(dev), x[kn].to(dev), x["w"].to(dev)
    gate = torch.full((wl.s_k,), 0.25, dtype=torch.float32, device=dev)
    i0, s0 = dsa.dsa_index_score_topk(q_idx, k_idx, w, wl.k_pools, chunk_q=256, want_scores=True)
    i1, s1 = dsa.dsa_index_score_topk_gated(q_idx, k_idx, gate, w, wl.k_pools, chunk_q=256,
                                            want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(i0, i1) and torch.equal(s0, s1)


# ---------------------------------------------------------------- small, every row

def test_tiny_workload_all_rows():
    run_case(inputs.WORKLOADS["tiny_s2048"])


@pytest.mark.parametrize("h_idx,d_idx", [(32, 128), (16, 96), (8, 64), (4, 128), (32, 96)])
def test_indexer_shapes_ragged(h_idx, d_idx):
    # chunks of 192 queries, a ragged last chunk and several 256-pool blocks;
    # k is small against the rows' lengths, so the early chunks are scored in
    # full and the later ones with error bounds and rescoring
    wl = inputs.custom(f"ragged_{h_idx}x{d_idx}", s_q=2500, s_k=2500, h_idx=h_idx, d_idx=d_idx,
                       k_pools=16, h=16, d=d_idx, idx_std=1 / math.sqrt(d_idx),
                       attn_std=1 / math.sqrt(d_idx), number=200 + h_idx + d_idx)
    run_case(wl, chunk_q=192)


def test_offset_queries_per_query_weights_and_tail():
    wl = inputs.custom("offset_tail", s_q=700, s_k=3003, q_pos0=2303, h_idx=32, d_idx=128,
                       k_pools=100, h=12, d=96, dv=64, n_tail=3, idx_std=0.1, number=301)
    run_case(wl, chunk_q=128, w_per_query=True)


@pytest.mark.parametrize("n_tail", [1, 2])
def test_partial_tails(n_tail):
    wl = inputs.custom(f"tail{n_tail}", s_q=300, s_k=300, h_idx=8, d_idx=64, k_pools=16, h=5,
                       d=64, dv=128, n_tail=n_tail, number=310 + n_tail)
    run_case(wl, chunk_q=64)


def test_k_covers_every_pool_equals_dense_attention():
    # with k >= P the selection is every eligible pool and the attention is
    # dense masked attention (section "Making Sparse Attention Actually Sparse")
    wl = inputs.custom("dense_equiv", s_q=520, s_k=520, h_idx=4, d_idx=64, k_pools=200, h=16,
                       d=128, n_tail=3, number=320)
    x, idx_g = run_case(wl, chunk_q=64)
    idx = idx_g.cpu().numpy()
    for t in range(520):
        n = min(t // 4, 130)
        assert np.array_equal(idx[t, :n], np.arange(n))


def test_k_equals_one_and_tiny_sequences():
    wl = inputs.custom("k1", s_q=130, s_k=130, h_idx=4, d_idx=64, k_pools=1, h=1, d=64,
                       number=330)
    run_case(wl, chunk_q=64)
    wl = inputs.custom("s3", s_q=3, s_k=3, h_idx=4, d_idx=64, k_pools=4, h=2, d=64, number=331)
    run_case(wl, chunk_q=64, check_scores=False)


def test_ties_resolve_to_lower_ids():
    wl = inputs.custom("ties", s_q=1100, s_k=1100, h_idx=8, d_idx=64, k_pools=37, h=4, d=64,
                       number=340)
    x = inputs.make_inputs(wl)
    # all weights zero: every score is +0 and the first k pools are kept
    x0 = dict(x)
    x0["w"] = torch.zeros_like(x["w"])
    _, idx0 = run_case(wl, chunk_q=64, x=x0, attention=False)
    idx0 = idx0.cpu().numpy()
    for t in range(wl.s_q):
        n = min(t // 4, wl.n_pools)
        m = min(n, wl.k_pools)
        assert np.array_equal(idx0[t, :m], np.arange(m)) and np.all(idx0[t, m:] == -1)
    # duplicated pools: pools 10..19 copy pools 0..9, so equal scores straddle the boundary
    x1 = dict(x)
    k = x["k_idx"].clone()
    for r in range(10):
        k[4 * (10 + r): 4 * (11 + r)] = k[4 * r: 4 * (r + 1)]
    k[200:1100] = (k[200:1100].float() * 0.25).to(torch.bfloat16)
    x1["k_idx"] = k
    _, idx1 = run_case(wl, chunk_q=64, x=x1, attention=False)
    # pools j and j + 10 have bit-identical pooled keys, hence identical
    # scores: whenever exactly one of them is kept it must be the lower id
    # (an exact tie lies inside the boundary band, so the oracle comparison
    # alone would accept the wrong copy as a swap)
    idx1 = idx1.cpu().numpy()
    straddles = 0
    for t in range(wl.s_q):
        kept = set(idx1[t].tolist())
        for j in range(10):
            if (j in kept) != (j + 10 in kept):
                straddles += 1
                assert j in kept, f"row {t}: the higher copy {j + 10} of pool {j} was kept"
    _say(f"  tie pairs split by the boundary: {straddles}")
    assert straddles > 100  # the case does exercise the rule (the oracle splits 530)


def test_large_row_paths_and_sampling():
    # rows longer than the LDS candidate list (4096 pools) take the sampled path;
    # a heavy-tied row forces the exact fallback
    wl = inputs.custom("long_rows", s_q=256, s_k=40000, q_pos0=39744, h_idx=16, d_idx=64,
                       k_pools=300, h=4, d=64, number=350)
    run_case(wl, rows=np.arange(0, 256, 3), chunk_q=128)
    x = inputs.make_inputs(wl, attention=False)
    x["w"] = torch.zeros_like(x["w"])
    _, idx0 = run_case(wl, rows=np.arange(0, 256, 17), chunk_q=128, x=x, attention=False,
                       check_scores=False)
    assert np.all(idx0.cpu().numpy() == np.arange(wl.k_pools)[None, :])


def test_largest_k_2048_pools():
    # the largest k the ABI accepts (2048 pools, 8192 attended tokens per
    # query), on rows longer than the LDS list (sampled threshold) and on rows
    # shorter than k (every pool, -1 padding)
    wl = inputs.custom("k2048", s_q=160, s_k=40000, q_pos0=39840, h_idx=32, d_idx=128,
                       k_pools=2048, h=16, d=128, idx_std=1 / math.sqrt(128), number=470)
    run_case(wl, rows=np.arange(0, 160, 5), chunk_q=64, check_scores=False)
    wl = inputs.custom("k2048_short", s_q=96, s_k=8200, q_pos0=8104, h_idx=16, d_idx=64,
                       k_pools=2048, h=8, d=64, n_tail=3, number=471)
    run_case(wl, rows=np.arange(0, 96, 7), chunk_q=64, check_scores=False)


def _host_topk_ids(scores, n, k):
    """Exact top-k of one row of fp32 scores by (-score, id), ascending ids,
    -1 padded: the selection rule restated on the host."""
    if n <= k:
        return np.concatenate([np.arange(n), np.full(k - n, -1)]).astype(np.int32)
    order = np.lexsort((np.arange(n), -scores[:n].astype(np.float64)))
    return np.sort(order[:k]).astype(np.int32)


@pytest.mark.parametrize("s_k,q_pos0,keys,k_pools", [
    (65536, 65344, "random", 512), (65536, 65344, "near_constant", 512),  # bounded, 16k pools
    (131072, 130880, "random", 512), (131072, 130880, "near_constant", 512),  # 32k pools
    (80192, 80000, "random", 512),                      # rows of 20k pools, scored in full
    (65536, 65344, "pool_constant", 512),  # every pooled key exactly bf16: no correction term
    (16448, 16256, "random", 64),  # bounded rows of 4064-4111 pools, sampled
    (12480, 12288, "random", 64),  # 96-wide heads, rows of 3072-3119 pools: whole short list,
                                   # then sampled
    (12480, 12288, "near_constant", 64),  # the short list overflows into the slow path
])
def test_selection_equals_exact_topk_of_full_scores(s_k, q_pos0, keys, k_pools):
    # The chunk buffer holds scores taken without the E4M3 correction; the
    # selection rescores only the pools its error bound cannot decide.  The
    # kept ids must be exactly the top-k of the full scores, which
    # dsa_index_scores returns (same MFMA sequence).  Near-constant keys put
    # nearly every pool within the bound of the threshold, so long rows
    # overflow the LDS list and take the slow path in global memory.  At
    # 80000 the chunk's rows are short enough to be scored in full, so the
    # selection works on final scores.  With the 4 keys of every pool equal,
    # each pooled key is exactly bf16 and every correction code is 0; the
    # chunk's scores still differ from the full ones by the rounding of a
    # different summation order, which the bound must cover.
    near_constant = keys == "near_constant"
    d_idx = 96 if s_k == 12480 else 128
    wl = inputs.custom("full_topk", s_q=192, s_k=s_k, q_pos0=q_pos0, h_idx=32, d_idx=d_idx,
                       k_pools=k_pools, h=16, d=128, idx_std=1 / math.sqrt(d_idx),
                       number=380 + {"random": 0, "near_constant": 1, "pool_constant": 2}[keys]
                       + (s_k - 65536) // 4096 + (k_pools != 512) * 1000 + (d_idx != 128) * 2000)
    x = inputs.make_inputs(wl, attention=False)
    if near_constant:
        rng = np.random.default_rng(7)
        base = rng.standard_normal(wl.d_idx).astype(np.float32) / np.float32(math.sqrt(wl.d_idx))
        noise = rng.standard_normal((wl.s_k, wl.d_idx)).astype(np.float32)
        x["k_idx"] = torch.from_numpy(base[None, :] * (1 + np.float32(0.01) * noise)).to(
            torch.bfloat16)
    if keys == "pool_constant":
        x["k_idx"] = x["k_idx"][0::4].repeat_interleave(4, dim=0)[:wl.s_k].contiguous()
    dev = torch.device("cuda")
    q_idx, k_idx, w = x["q_idx"].to(dev), x["k_idx"].to(dev), x["w"].to(dev)
    idx, sc = dsa.dsa_index_score_topk(q_idx, k_idx, w, wl.k_pools, q_pos0=wl.q_pos0,
                                       chunk_q=64, want_scores=True)
    idx_b, _ = dsa.dsa_index_score_topk(q_idx, k_idx, w, wl.k_pools, q_pos0=wl.q_pos0,
                                        chunk_q=64)
    full = dsa.dsa_index_scores(q_idx, k_idx, w, row0=0, n_rows=wl.s_q, q_pos0=wl.q_pos0)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_b), "ids without score_out differ from ids with it"
    idx, sc, full = idx.cpu().numpy(), sc.cpu().numpy(), full.cpu().numpy()
    for i in range(wl.s_q):
        n = min((wl.q_pos0 + i) // 4, wl.n_pools)
        want = _host_topk_ids(full[i], n, wl.k_pools)
        assert np.array_equal(idx[i], want), f"row {i}: ids differ from the full-score top-k"
        sel = want >= 0
        assert np.array_equal(sc[i][sel].view(np.uint32), full[i][want[sel]].view(np.uint32)), \
            f"row {i}: selected scores differ from the full scores"
    if near_constant:
        # and against the oracle, within the parity rules
        run_case(wl, rows=np.arange(0, wl.s_q, 16), chunk_q=64, x=x, attention=False,
                 check_scores=False)


@pytest.mark.parametrize("h_idx,d_idx,scales,s_k", [
    (32, 96, (1.0, 1.0), 20000), (32, 128, (-0.5, 1.0), 20000), (4, 64, (-2.0, 0.5), 20000),
    (8, 96, (1.0, 3.0), 20000),
    # rows of about 3000 pools: sampled, though they would fit the list
    (32, 96, (1.0, 1.0), 12200),
    # rows of about 2000 pools: the whole row goes to the list
    (32, 128, (1.0, 1.0), 8200),
])
def test_fp8_selection_equals_exact_topk_of_dense_scores(h_idx, d_idx, scales, s_k):
    # The fp8 indexer selects on final scores: the chunk path's ids and kept
    # scores must be exactly the top-k of the dense scores (same kernel,
    # masked stores), for both signs of q_scale * k_scale, with rows longer
    # than the LDS list (sampled threshold) and shorter ones.
    wl = inputs.custom(f"fp8_topk_{h_idx}x{d_idx}_{s_k}", s_q=192, s_k=s_k, q_pos0=s_k - 192,
                       h_idx=h_idx, d_idx=d_idx, k_pools=300, h=16, d=128, fp8=True,
                       number=440 + h_idx + d_idx + (s_k != 20000) * s_k // 100)
    _say(f"[case] {wl.name} scales={scales}")
    x = inputs.make_inputs(wl, attention=False)
    dev = torch.device("cuda")
    q8, k8, w = x["q_idx8"].to(dev), x["k_idx8"].to(dev), x["w"].to(dev)
    kw = dict(q_scale=torch.tensor([scales[0]], dtype=torch.float32, device=dev),
              k_scale=torch.tensor([scales[1]], dtype=torch.float32, device=dev))
    idx, sc = dsa.dsa_index_score_topk(q8, k8, w, wl.k_pools, q_pos0=wl.q_pos0, chunk_q=64,
                                       want_scores=True, **kw)
    idx_b, _ = dsa.dsa_index_score_topk(q8, k8, w, wl.k_pools, q_pos0=wl.q_pos0, chunk_q=64,
                                        **kw)
    full = dsa.dsa_index_scores(q8, k8, w, row0=0, n_rows=wl.s_q, q_pos0=wl.q_pos0, **kw)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_b), "ids without score_out differ from ids with it"
    idx, sc, full = idx.cpu().numpy(), sc.cpu().numpy(), full.cpu().numpy()
    for i in range(wl.s_q):
        n = min((wl.q_pos0 + i) // 4, wl.n_pools)
        want = _host_topk_ids(full[i], n, wl.k_pools)
        assert np.array_equal(idx[i], want), f"row {i}: ids differ from the dense-score top-k"
        sel = want >= 0
        assert np.array_equal(sc[i][sel].view(np.uint32), full[i][want[sel]].view(np.uint32)), \
            f"row {i}: kept scores differ from the dense scores"


def test_deterministic_bitwise():
    wl = inputs.custom("determinism", s_q=1500, s_k=1500, h_idx=32, d_idx=128, k_pools=64,
                       h=16, d=128, number=360)
    x = inputs.make_inputs(wl)
    dev = torch.device("cuda")
    a = [t.to(dev) for t in (x["q_idx"], x["k_idx"], x["w"], x["q"], x["k"], x["v"])]
    outs = []
    for _ in range(2):
        idx, sc = dsa.dsa_index_score_topk(a[0], a[1], a[2], 64, want_scores=True)
        o, lse = dsa.dsa_sparse_attn_fwd(a[3], a[4], a[5], idx, want_lse=True)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (idx, sc, o, lse)])
    for u, v in zip(*outs):
        assert torch.equal(u.view(torch.uint8) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.uint8) if v.dtype == torch.bfloat16 else v)


def test_k_and_v_may_alias():
    wl = inputs.custom("kv_alias", s_q=400, s_k=400, h_idx=4, d_idx=64, k_pools=20, h=8, d=64,
                       number=370)
    x = inputs.make_inputs(wl)
    x["v"] = x["k"]
    run_case(wl, chunk_q=64, x=x)


def test_hardware_e4m3_conversion_matches_the_format_definition():
    # The query packing encodes its scaled rows (bf16 values times a power of
    # two, |x| <= 448) with v_cvt_pk_fp8_f32 and decodes them with
    # v_cvt_f32_fp8.  Both against the oracle's E4M3 definition (nearest
    # value, ties to the even mantissa, sign kept): every bf16 value up to
    # 448, float32 subnormals, and random float32 values up to 448.
    import ctypes
    import os
    lib = ctypes.CDLL(os.path.join(os.path.dirname(dsa.__file__), "libdsa_peaks.so"))
    lib.dsa_probe_e4m3.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_void_p]
    bf = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(977)
    sub = (rng.integers(1, 1 << 23, 2000, dtype=np.uint32) |
           (rng.integers(0, 2, 2000, dtype=np.uint32) << 31)).view(np.float32)
    rnd = rng.uniform(-448.0, 448.0, 100000).astype(np.float32)
    x = np.concatenate([bf, sub, rnd])
    x = x[np.isfinite(x) & (np.abs(x) <= 448.0)]
    _say(f"[case] hardware E4M3 round trip of {len(x)} floats")
    dev = torch.device("cuda")
    xd = torch.from_numpy(x).to(dev)
    code = torch.empty(len(x), dtype=torch.uint8, device=dev)
    val = torch.empty(len(x), dtype=torch.float32, device=dev)
    rc = lib.dsa_probe_e4m3(xd.data_ptr(), code.data_ptr(), val.data_ptr(), len(x),
                            torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    code, val = code.cpu().numpy(), val.cpu().numpy()
    want = np.array([oracle.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    bad = np.flatnonzero(code != want)
    assert bad.size == 0, (f"{bad.size} codes differ, first x={x[bad[0]]!r}: "
                           f"hardware 0x{code[bad[0]]:02x}, definition 0x{want[bad[0]]:02x}")
    dec = np.array([oracle.e4m3_value(int(c)) for c in range(256)], dtype=np.float64)
    assert np.array_equal(val.astype(np.float64), dec[code])


@pytest.mark.parametrize("h_idx,d_idx,scales", [
    (32, 96, (1.0, 1.0)), (32, 128, (0.5, 2.0)), (4, 64, (1.0, 1.0)), (16, 96, (-1.5, 0.25)),
    (8, 128, (3.0, 1.0)),
])
def test_fp8_indexer(h_idx, d_idx, scales):
    # section "Making Sparse Attention Actually Sparse" (NoPE heads): the E4M3
    # indexer with per-pool power-of-two re-quantisation of the pooled keys
    wl = inputs.custom(f"fp8_{h_idx}x{d_idx}", s_q=2100, s_k=2100, h_idx=h_idx, d_idx=d_idx,
                       k_pools=48, h=16, d=96, n_tail=3, fp8=True, number=400 + h_idx + d_idx)
    run_case(wl, chunk_q=256, fp8=True, scales=scales, attention=(h_idx == 32))


# ---------------------------------------------------------------- the page's workloads

def _full_size_rows(wl, n, fp8=False, chunk_q=0):
    """A strided sample of n rows plus the first and last row of every
    selection launch of the default (or given) chunking."""
    _, cq = dsa.dsa_index_workspace_size(wl.s_q, wl.s_k, wl.h_idx, wl.d_idx, wl.k_pools, 4,
                                         chunk_q, dsa.DSA_FP8_E4M3 if fp8 else dsa.DSA_BF16)
    ends = [r for c0 in range(0, wl.s_q, cq) for r in (c0, min(wl.s_q, c0 + cq) - 1)]
    rows = inputs.sample_rows(wl.s_q, n, extra=ends)
    _say(f"[rows] {wl.name}: {len(rows)} rows, chunks of {cq} queries "
         f"({(wl.s_q + cq - 1) // cq} selection launches, each with checked rows)")
    return rows


def test_workload_s32k_sampled():
    wl = inputs.WORKLOADS["s32k"]
    run_case(wl, rows=_full_size_rows(wl, 384))


def test_workload_s32k_chunks_of_256_sampled():
    # the workload as described: queries scored and selected in chunks of 256
    wl = inputs.WORKLOADS["s32k"]
    run_case(wl, rows=_full_size_rows(wl, 256, chunk_q=256), chunk_q=256, tag="chunks of 256")


@pytest.mark.slow
def test_workload_s128k_sampled():
    wl = inputs.WORKLOADS["s128k"]
    run_case(wl, rows=_full_size_rows(wl, 2048))


@pytest.mark.slow
def test_workload_s128k_gated_sampled():
    # the headline shape with per-token k-pool gates (bf16 indexer)
    wl = inputs.WORKLOADS["s128k"]
    run_case(wl, rows=_full_size_rows(wl, 256), attention=False, gate=inputs.make_gates(wl))


@pytest.mark.slow
def test_workload_nope_s64k_fp8_gated_sampled():
    wl = inputs.WORKLOADS["nope_s64k"]
    run_case(wl, rows=_full_size_rows(wl, 256, fp8=True), attention=False, fp8=True,
             gate=inputs.make_gates(wl))


@pytest.mark.slow
def test_workload_nope_s64k_sampled():
    wl = inputs.WORKLOADS["nope_s64k"]
    run_case(wl, rows=_full_size_rows(wl, 512))


@pytest.mark.slow
def test_workload_nope_s64k_fp8_sampled():
    wl = inputs.WORKLOADS["nope_s64k"]
    run_case(wl, rows=_full_size_rows(wl, 512, fp8=True), fp8=True)


@pytest.mark.slow
def test_workload_share_1m_sampled():
    # at least one checked row in every selection launch (1536-query chunks).
    # The oracle needs about 2 s of one core per row at this size, so the
    # default run checks a strided 128 plus the chunk ends; DSA_PARITY_WIDE=1
    # checks 2048 strided rows plus the ends (several minutes of CPU).
    wl = inputs.WORKLOADS["share_1m"]
    n = 2048 if os.environ.get("DSA_PARITY_WIDE") == "1" else 128
    run_case(wl, rows=_full_size_rows(wl, n), tag="wide" if n > 128 else "")
