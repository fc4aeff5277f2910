"""Pins of the CPU oracle against things other than itself (no GPU).

Method source: SkyRL blog "Scaling Training to 1M Token Context on
GLM-5.3-Flash" -- section "DeepSeek Sparse Attention (DSA) Optimizations"
(rate each 4-token pool before the query, attend to the chosen tokens alone),
"Making Sparse Attention Actually Sparse" (2,051 keys), "Over Time: Chunking"
(fp32 scores) and "Across GPUs: Sharding" (int32 pool ids).  The page prints
no worked example, so the pins are: hand-derived closed forms on tiny inputs,
published number-format definitions (bfloat16, OCP E4M3) checked against
torch's own casts, brute force by a different route (tests/brute.py), the
special case that reduces to dense masked attention (torch SDPA), and
invariants.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle
from long_context_sparse_dsa_amd import inputs
import brute


def bf(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)


# ---------------------------------------------------------------- formats

def test_bf16_decode_known_patterns():
    assert oracle.bf16_value(0x3F80) == 1.0
    assert oracle.bf16_value(0xC000) == -2.0
    assert oracle.bf16_value(0x3E00) == 0.125
    assert oracle.bf16_value(0x0001) == 2.0 ** -133          # smallest subnormal
    assert oracle.bf16_value(0x7F7F) == (2 - 2 ** -7) * 2.0 ** 127
    assert oracle.bf16_value(0x8000) == 0.0 and math.copysign(1, oracle.bf16_value(0x8000)) < 0


def test_bf16_decode_matches_torch_on_all_finite_patterns():
    bits = np.arange(0, 1 << 16, 97, dtype=np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for b, ref in zip(bits, t):
        v = oracle.bf16_value(int(b))
        if np.isnan(ref):
            assert np.isnan(v)
        else:
            assert v == ref


def test_e4m3_table_values_from_the_ocp_definition():
    assert oracle.e4m3_value(0x38) == 1.0             # exponent 7 = bias
    assert oracle.e4m3_value(0x7E) == 448.0           # largest finite
    assert oracle.e4m3_value(0xFE) == -448.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6       # smallest normal
    assert oracle.e4m3_value(0x01) == 2.0 ** -9       # smallest subnormal
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert math.isnan(oracle.e4m3_value(0x7F))
    assert math.isnan(oracle.e4m3_value(0xFF))


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c, r in zip(codes, ref):
        v = oracle.e4m3_value(int(c))
        assert (np.isnan(v) and np.isnan(r)) or v == r


def test_e4m3_encode_ties_and_saturation():
    assert oracle.e4m3_encode(1.0) == 0x38
    assert oracle.e4m3_encode(1.0625) == 0x38          # tie between 1.0 and 1.125 -> even
    assert oracle.e4m3_encode(1.1875) == 0x3A          # tie between 1.125 and 1.25 -> even
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00      # tie between 0 and 2^-9 -> 0
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie between 2^-9 and 2^-8 -> even
    assert oracle.e4m3_encode(460.0) == 0x7E           # saturates
    assert oracle.e4m3_encode(-1e6) == 0xFE
    assert oracle.e4m3_encode(-1.0) == 0xB8


def test_e4m3_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    x = x[np.abs(x) <= 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    # torch may keep the sign of an underflow to zero; compare values
    gv = np.array([oracle.e4m3_value(int(c)) for c in got])
    rv = torch.from_numpy(ref).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(gv, rv)


# ---------------------------------------------------------------- hand example

# Three pools of 4 tokens, D_I = 2, H_I = 2.
#   pool 0 rows [1,0],[2,0],[3,0],[2,4]    -> kbar0 = [2, 1]
#   pool 1 rows [0,1],[0,1],[-4,1],[0,1]   -> kbar1 = [-1, 1]
#   pool 2 rows [1,-2] x 4                 -> kbar2 = [1, -2]
# Query heads h0 = [1, 1], h1 = [0.5, -1].
#   dots h0: [3, 0, -1]; h1: [0, -1.5, 2.5]
# w = [1, 2]:  s = [1*3 + 2*0, 0 + 0, 0 + 2*2.5] = [3, 0, 5]
# w = [1, -1]: s = [3, 0, -2.5]
HAND_K = [[1, 0], [2, 0], [3, 0], [2, 4],
          [0, 1], [0, 1], [-4, 1], [0, 1],
          [1, -2], [1, -2], [1, -2], [1, -2]]
HAND_Q = [[1, 1], [0.5, -1]]


def _hand(q_pos_list, w):
    k = bf(HAND_K)
    q = bf([HAND_Q] * len(q_pos_list))
    return q, k, torch.tensor(w, dtype=torch.float32)


def test_hand_pooled_keys():
    kbar = oracle.pool_keys(bf(HAND_K))
    assert np.array_equal(kbar, [[2, 1], [-1, 1], [1, -2]])


def test_hand_scores_and_causality():
    # one query per position; rows map to positions q_pos0 + row
    q, k, w = _hand(range(13), [1.0, 2.0])
    s = oracle.index_scores(q, k, w, q_pos0=0)
    inf = -np.inf
    expect = {0: [inf, inf, inf], 3: [inf, inf, inf],      # no complete pool before t
              4: [3, inf, inf], 7: [3, inf, inf],          # pool 1 holds token 7 itself
              8: [3, 0, inf], 11: [3, 0, inf],
              12: [3, 0, 5]}
    for t, e in expect.items():
        assert np.array_equal(s[t], np.array(e, dtype=np.float32)), (t, s[t])


def test_hand_scores_negative_weight_applies_after_relu():
    q, k, w = _hand([12], [1.0, -1.0])
    s = oracle.index_scores(q, k, w, q_pos0=12)
    assert np.array_equal(s[0], np.array([3, 0, -2.5], dtype=np.float32))


def test_hand_topk():
    q, k, w = _hand(range(13), [1.0, 2.0])
    idx, sc = oracle.index_topk(q, k, w, k_pools=2, q_pos0=0)
    assert idx[12].tolist() == [0, 2] and sc[12].tolist() == [3.0, 5.0]
    assert idx[8].tolist() == [0, 1]             # n(t) <= k: every eligible pool
    assert idx[5].tolist() == [0, -1]
    assert idx[2].tolist() == [-1, -1] and np.all(np.isneginf(sc[2]))
    idx1, _ = oracle.index_topk(q, k, w, k_pools=1, q_pos0=0)
    assert idx1[12].tolist() == [2] and idx1[9].tolist() == [0]


def test_hand_q_pos0_offsets_positions():
    q, k, w = _hand([12], [1.0, 2.0])
    s = oracle.index_scores(q, k, w, q_pos0=12)
    assert np.array_equal(s[0], np.array([3, 0, 5], dtype=np.float32))
    s = oracle.index_scores(q, k, w, q_pos0=9)
    assert np.array_equal(s[0], np.array([3, 0, -np.inf], dtype=np.float32))


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("s,h_idx,d_idx,k_pools,w_per_query,q_pos0", [
    (8, 4, 64, 1, False, 0), (13, 4, 64, 2, False, 0), (64, 8, 32, 4, True, 0),
    (256, 32, 128, 16, False, 0), (301, 4, 96, 8, True, 40),
])
def test_scores_and_selection_match_brute_force(s, h_idx, d_idx, k_pools, w_per_query, q_pos0):
    wl = inputs.custom(s_q=s - q_pos0 if q_pos0 else s, s_k=s, q_pos0=q_pos0, h_idx=h_idx,
                       d_idx=d_idx, k_pools=k_pools, idx_std=0.125)
    x = inputs.make_inputs(wl, seed=11 + s, attention=False, w_per_query=w_per_query)
    got = oracle.index_scores(x["q_idx"], x["k_idx"], x["w"], q_pos0=q_pos0)
    ref = brute.raw_token_scores(x["q_idx"], x["k_idx"], x["w"], q_pos0=q_pos0)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got))
    # the two fp64 roads differ only by summation order: at most 1 fp32 ulp
    assert np.all(np.abs(got[fin] - ref[fin]) <= np.spacing(np.abs(ref[fin])) + 1e-30)
    idx, sc = oracle.index_topk(x["q_idx"], x["k_idx"], x["w"], k_pools, q_pos0=q_pos0)
    for r in range(wl.s_q):
        n = min((q_pos0 + r) // 4, wl.n_pools)
        expect = brute.rank_select(got[r], n, k_pools)
        assert np.array_equal(idx[r], expect), r
        sel = idx[r][idx[r] >= 0]
        assert np.array_equal(sc[r][: len(sel)], got[r][sel])


def test_all_zero_weights_select_lowest_ids():
    wl = inputs.custom(s_q=64, s_k=64, h_idx=4, d_idx=64, k_pools=3)
    x = inputs.make_inputs(wl, seed=3, attention=False)
    w = torch.zeros(4)
    idx, sc = oracle.index_topk(x["q_idx"], x["k_idx"], w, 3)
    assert idx[63].tolist() == [0, 1, 2] and np.all(sc[63] == 0)
    assert np.all(np.signbit(sc[63]) == False)  # +0, never -0


def test_duplicate_pools_tie_to_lower_index():
    wl = inputs.custom(s_q=40, s_k=40, h_idx=4, d_idx=64, k_pools=2)
    x = inputs.make_inputs(wl, seed=5, attention=False)
    s = oracle.index_scores(x["q_idx"], x["k_idx"], x["w"], rows=[39])[0]
    best = int(np.argmax(s))
    k = x["k_idx"].clone()
    k[8:12] = x["k_idx"][4 * best: 4 * best + 4]    # pools 2 and 7 copy the best pool
    k[28:32] = x["k_idx"][4 * best: 4 * best + 4]
    s = oracle.index_scores(x["q_idx"], k, x["w"], rows=[39])[0]
    assert s[2] == s[7] == s.max()
    ties = [p for p in range(9) if s[p] == s.max()]
    idx, _ = oracle.index_topk(x["q_idx"], k, x["w"], 1, rows=[39])
    assert idx[0].tolist() == [ties[0]] and ties[0] <= 2
    idx, _ = oracle.index_topk(x["q_idx"], k, x["w"], len(ties), rows=[39])
    assert idx[0].tolist() == ties


def test_metamorphic_scaling_and_head_permutation():
    wl = inputs.custom(s_q=200, s_k=200, h_idx=8, d_idx=64, k_pools=8)
    x = inputs.make_inputs(wl, seed=9, attention=False)
    rows = [50, 123, 199]
    s0 = oracle.index_scores(x["q_idx"], x["k_idx"], x["w"], rows=rows)
    s2 = oracle.index_scores(x["q_idx"], x["k_idx"], 2 * x["w"], rows=rows)
    assert np.array_equal(np.where(np.isfinite(s0), 2 * s0, s0), s2)
    q2 = (x["q_idx"].float() * 2).to(torch.bfloat16)
    s2q = oracle.index_scores(q2, x["k_idx"], x["w"], rows=rows)
    assert np.array_equal(s2q, s2)
    perm = torch.randperm(8, generator=torch.Generator().manual_seed(1))
    sp = oracle.index_scores(x["q_idx"][:, perm], x["k_idx"], x["w"][perm], rows=rows)
    fin = np.isfinite(s0)
    assert np.all(np.abs(sp[fin] - s0[fin]) <= np.spacing(np.abs(s0[fin])))
    i0, _ = oracle.index_topk(x["q_idx"], x["k_idx"], x["w"], 8, rows=rows)
    i2, _ = oracle.index_topk(x["q_idx"], x["k_idx"], 2 * x["w"], 8, rows=rows)
    assert np.array_equal(i0, i2)


def test_selection_is_strictly_causal_and_ascending():
    wl = inputs.custom(s_q=500, s_k=500, h_idx=4, d_idx=64, k_pools=16)
    x = inputs.make_inputs(wl, seed=21, attention=False)
    idx, _ = oracle.index_topk(x["q_idx"], x["k_idx"], x["w"], 16)
    for t in range(500):
        row = idx[t]
        v = row[row >= 0]
        assert np.all(4 * v + 3 < t)
        assert np.all(np.diff(v) > 0)
        assert np.all(row[len(v):] == -1)
        assert len(v) == min(t // 4, 16)


# ---------------------------------------------------------------- attention

def _attn_case(s, h=4, d=32, dv=None, q_pos0=0, seed=0):
    wl = inputs.custom(s_q=s - q_pos0, s_k=s, q_pos0=q_pos0, h=h, d=d, dv=dv, h_idx=4, d_idx=32,
                       k_pools=4)
    return wl, inputs.make_inputs(wl, seed=seed, indexer=False)


@pytest.mark.parametrize("n_tail", [0, 3])
def test_attention_with_every_pool_equals_dense_masked_attention(n_tail):
    wl, x = _attn_case(67, h=4, d=32, dv=48, seed=1)
    P = wl.n_pools
    rows = np.arange(wl.s_q)
    idx = np.full((len(rows), P), -1, dtype=np.int32)
    for r in rows:
        n = min(r // 4, P)
        idx[r, :n] = np.arange(n)
    scale = float(np.float32(1 / math.sqrt(32)))
    o, lse = oracle.sparse_attn(x["q"], x["k"], x["v"], idx, P, rows=rows, n_tail=n_tail,
                                scale=scale)
    ro, rlse = brute.dense_attention(x["q"], x["k"], x["v"], 0, rows, n_tail == 3, scale)
    for r in rows:
        visible = r if n_tail == 3 else 4 * (r // 4)
        if visible == 0:
            assert np.all(o[r] == 0) and np.all(np.isneginf(lse[r]))
        else:
            np.testing.assert_allclose(o[r], ro[r], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[r], rlse[r], rtol=0, atol=1e-12)


def test_attention_partial_tail_lengths():
    wl, x = _attn_case(40, seed=2)
    rows = [37, 38, 39]                   # t mod 4 = 1, 2, 3
    idx = np.array([[0, 3, -1, -1]] * 3, dtype=np.int32)
    for n_tail, expect in [(1, [9, 9, 9]), (2, [9, 10, 10]), (3, [9, 10, 11])]:
        counts = [oracle.token_count(idx[i:i + 1], 0, 40, 4, [r], n_tail) for i, r in enumerate(rows)]
        assert counts == expect
    # the tail tokens are the ones right before t: compare with an explicit set
    o, _ = oracle.sparse_attn(x["q"], x["k"], x["v"], idx, 4, rows=rows, n_tail=2, scale=0.25)
    q = x["q"].double(); k = x["k"].double(); v = x["v"].double()
    for i, r in enumerate(rows):
        toks = [0, 1, 2, 3, 12, 13, 14, 15] + list(range(max(36, r - 2), r))
        lg = (q[r] @ k[toks].T) * 0.25
        ref = torch.softmax(lg, dim=-1) @ v[toks]
        np.testing.assert_allclose(o[i], ref.numpy(), rtol=0, atol=1e-12)


def test_attention_closed_forms():
    wl, x = _attn_case(64, h=2, d=32, seed=3)
    rows = [40, 63]
    idx = np.array([[1, 4, 6, -1], [0, 2, 9, 14]], dtype=np.int32)
    # all value rows equal c  ->  o = c
    v = torch.full_like(x["v"], 0.375)
    o, _ = oracle.sparse_attn(x["q"], x["k"], v, idx, 4, rows=rows)
    np.testing.assert_allclose(o, 0.375, rtol=1e-14, atol=0)
    # all key rows equal  ->  uniform weights, o = mean of v over T(t)
    k = x["k"][:1].expand_as(x["k"]).contiguous()
    o, lse = oracle.sparse_attn(x["q"], k, x["v"], idx, 4, rows=rows)
    vd = x["v"].double().numpy()
    for i, row in enumerate(idx):
        toks = [4 * p + u for p in row if p >= 0 for u in range(4)]
        np.testing.assert_allclose(o[i], np.broadcast_to(vd[toks].mean(0), o[i].shape),
                                   rtol=0, atol=1e-13)
        # o lies inside the per-column range of v over T(t)
    o, _ = oracle.sparse_attn(x["q"], x["k"], x["v"], idx, 4, rows=rows)
    for i, row in enumerate(idx):
        toks = [4 * p + u for p in row if p >= 0 for u in range(4)]
        assert np.all(o[i] >= vd[toks].min(0) - 1e-12) and np.all(o[i] <= vd[toks].max(0) + 1e-12)


def test_attention_rejects_malformed_index_rows():
    wl, x = _attn_case(64, seed=4)
    for bad in ([3, 1, -1, -1],       # not ascending
                [0, 0, -1, -1],       # duplicate
                [0, -1, 2, -1],       # id after padding
                [0, 15, -1, -1],      # pool 15 holds tokens 60..63 >= t
                [-2, -1, -1, -1]):
        with pytest.raises(RuntimeError):
            oracle.sparse_attn(x["q"], x["k"], x["v"], np.array([bad], dtype=np.int32), 4,
                               rows=[60])


# ---------------------------------------------------------------- fp8 indexer

def _fp8(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn)


def test_fp8_pool_requantisation_hand_example():
    # pool rows [1, 2], [1, 2], [1, 2], [1, 2.5]: mean [1, 2.125]; amax 2.125
    # smallest e with 2.125 <= 448 * 2^e is e = -7; scaled mean [128, 272];
    # 272 lies halfway between 256 and 288 -> ties to even -> 256.
    k8 = _fp8([[1, 2], [1, 2], [1, 2], [1, 2.5]])
    codes, exps = oracle.pool_keys_fp8(k8)
    assert exps.tolist() == [-7]
    assert [oracle.e4m3_value(int(c)) for c in codes[0]] == [128.0, 256.0]


@pytest.mark.parametrize("amax,e", [(448.0, 0), (224.0, -1), (240.0, 0), (0.5, -9), (0.0, 0)])
def test_fp8_pool_exponent_rule(amax, e):
    row = [amax, -amax / 2]
    k8 = _fp8([row] * 4)
    assert oracle.e4m3_value(int(k8.view(torch.uint8)[0, 0])) == amax   # exact in E4M3
    _, exps = oracle.pool_keys_fp8(k8)
    assert exps.tolist() == [e]


def test_fp8_scores_hand_example():
    # pool 0 = HAND pool with E4M3-exact values; q heads in E4M3 too
    k8 = _fp8(HAND_K)
    q8 = _fp8([HAND_Q])
    w = torch.tensor([1.0, 2.0])
    codes, exps = oracle.pool_keys_fp8(k8)
    kb = np.array([[oracle.e4m3_value(int(c)) for c in row] for row in codes]) * \
        np.exp2(exps.astype(np.float64))[:, None]
    assert np.array_equal(kb, [[2, 1], [-1, 1], [1, -2]])     # these means are E4M3-exact
    s = oracle.index_scores_fp8(q8, k8, w, q_scale=0.5, k_scale=4.0, q_pos0=12)
    assert np.array_equal(s[0], np.array([6, 0, 10], dtype=np.float32))   # 2x the bf16 case


def test_fp8_scores_close_to_exact_scores():
    wl = inputs.custom(s_q=300, s_k=300, h_idx=8, d_idx=96, k_pools=8, fp8=True)
    x = inputs.make_inputs(wl, seed=17, attention=False)
    rows = [150, 299]
    s8 = oracle.index_scores_fp8(x["q_idx8"], x["k_idx8"], x["w"], rows=rows)
    qd = x["q_idx8"].float().to(torch.bfloat16)   # E4M3 values are bf16-exact
    kd = x["k_idx8"].float().to(torch.bfloat16)
    s = oracle.index_scores(qd, kd, x["w"], rows=rows)
    fin = np.isfinite(s)
    # re-quantising the pooled key costs ~ 2^-4 relative per element
    err = np.abs(s8[fin] - s[fin]) / (np.abs(s[fin]).max())
    assert err.max() < 0.06


# ---------------------------------------------------------------- gated pooling
# section "DSA: Gather by Token Position": each key of a pool is scaled by its
# own k-pool gate score before the pool is formed.  Reading: kbar_p = sum_r g[4p+r] k[4p+r] with caller-normalised
# gates; no gates means the mean.

def test_gated_pooling_with_quarter_gates_is_the_mean():
    wl = inputs.custom(s_q=96, s_k=96, h_idx=8, d_idx=64, k_pools=4, fp8=True)
    x = inputs.make_inputs(wl, seed=31, attention=False)
    g = np.full(wl.s_k, 0.25, dtype=np.float32)
    assert np.array_equal(oracle.pool_keys(x["k_idx"], gate=g), oracle.pool_keys(x["k_idx"]))
    c0, e0 = oracle.pool_keys_fp8(x["k_idx8"])
    c1, e1 = oracle.pool_keys_fp8(x["k_idx8"], gate=g)
    assert np.array_equal(c0, c1) and np.array_equal(e0, e1)
    i0, s0 = oracle.index_topk(x["q_idx"], x["k_idx"], x["w"], 4)
    i1, s1 = oracle.index_topk(x["q_idx"], x["k_idx"], x["w"], 4, gate=g)
    assert np.array_equal(i0, i1) and np.array_equal(s0, s1)


def test_gated_pooling_hand_example():
    # pool 0 rows of HAND_K with gates [0.5, 0.25, 0.125, 0.125]
    k = bf(HAND_K)
    g = np.array([0.5, 0.25, 0.125, 0.125] + [0.25] * 8, dtype=np.float32)
    kb = oracle.pool_keys(k, gate=g)
    rows = np.array(HAND_K[:4], dtype=np.float64)
    assert np.array_equal(kb[0], (g[:4, None] * rows).sum(axis=0))
    assert np.array_equal(kb[1:], oracle.pool_keys(k)[1:])


def test_gated_pooling_one_hot_gates_pick_a_token():
    wl = inputs.custom(s_q=64, s_k=64, h_idx=4, d_idx=64, k_pools=2, fp8=True)
    x = inputs.make_inputs(wl, seed=33, attention=False)
    for r0 in range(4):
        g = np.zeros(wl.s_k, dtype=np.float32)
        g[r0::4] = 1.0
        kb = oracle.pool_keys(x["k_idx"], gate=g)
        assert np.array_equal(kb, x["k_idx"][r0::4].to(torch.float64).numpy())
        # fp8: the pooled value is the token's own code value; re-quantising
        # it with a power-of-two scale reproduces it exactly
        codes, exps = oracle.pool_keys_fp8(x["k_idx8"], gate=g)
        vals = np.array([[oracle.e4m3_value(int(c)) for c in row] for row in codes])
        got = vals * np.exp2(exps.astype(np.float64))[:, None]
        assert np.array_equal(got, x["k_idx8"][r0::4].to(torch.float64).numpy())


@pytest.mark.parametrize("s,h_idx,d_idx,k_pools,q_pos0", [(64, 4, 64, 4, 0), (301, 8, 96, 8, 40)])
def test_gated_scores_and_selection_match_brute_force(s, h_idx, d_idx, k_pools, q_pos0):
    wl = inputs.custom(s_q=s - q_pos0, s_k=s, q_pos0=q_pos0, h_idx=h_idx, d_idx=d_idx,
                       k_pools=k_pools, idx_std=0.125)
    x = inputs.make_inputs(wl, seed=41 + s, attention=False, w_per_query=True)
    g = inputs.make_gates(wl, seed=41 + s)
    got = oracle.index_scores(x["q_idx"], x["k_idx"], x["w"], q_pos0=q_pos0, gate=g)
    ref = brute.raw_token_scores(x["q_idx"], x["k_idx"], x["w"], q_pos0=q_pos0, gate=g)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got))
    assert np.all(np.abs(got[fin] - ref[fin]) <= np.spacing(np.abs(ref[fin])) + 1e-30)
    # the gates matter: mean pooling gives different scores
    mean = oracle.index_scores(x["q_idx"], x["k_idx"], x["w"], q_pos0=q_pos0)
    assert not np.array_equal(mean[fin], got[fin])
    idx, _ = oracle.index_topk(x["q_idx"], x["k_idx"], x["w"], k_pools, q_pos0=q_pos0, gate=g)
    for r in range(wl.s_q):
        n = min((q_pos0 + r) // 4, wl.n_pools)
        assert np.array_equal(idx[r], brute.rank_select(got[r], n, k_pools)), r


def test_gated_scores_scale_with_the_gates():
    wl = inputs.custom(s_q=128, s_k=128, h_idx=8, d_idx=64, k_pools=4, fp8=True)
    x = inputs.make_inputs(wl, seed=43, attention=False)
    g = inputs.make_gates(wl, seed=43)
    rows = [60, 127]
    s1 = oracle.index_scores(x["q_idx"], x["k_idx"], x["w"], rows=rows, gate=g)
    s2 = oracle.index_scores(x["q_idx"], x["k_idx"], x["w"], rows=rows, gate=2 * g.numpy())
    assert np.array_equal(np.where(np.isfinite(s1), 2 * s1, s1), s2)
    # fp8: doubling the gates doubles the pooled values; the power-of-two
    # re-quantisation keeps the codes and moves the exponent by one
    c1, e1 = oracle.pool_keys_fp8(x["k_idx8"], gate=g)
    c2, e2 = oracle.pool_keys_fp8(x["k_idx8"], gate=2 * g.numpy())
    assert np.array_equal(c1, c2) and np.array_equal(e2, e1 + 1)


def test_gates_are_normalised_per_pool():
    wl = inputs.custom(s_q=40, s_k=42, h_idx=4, d_idx=64, k_pools=2)
    g = inputs.make_gates(wl, seed=5).numpy()
    sums = g[:40].reshape(-1, 4).sum(axis=1, dtype=np.float64)
    assert np.all(np.abs(sums - 1.0) < 1e-6) and np.all(g[:40] > 0) and np.all(g[40:] == 0)


# ---------------------------------------------------------------- memory model

def test_unchunked_indexer_memory_matches_the_page():
    # section "Over Time: Chunking": 64 GiB at 32k, about 1 TiB at 128k for the
    # unchunked score buffer.  Both equal 2 copies x 4 B x S x S/4 x 32 heads.
    def unchunked(s):
        return 2 * 4 * s * (s // 4) * 32
    assert unchunked(32768) == 64 * 2 ** 30
    assert unchunked(131072) == 2 ** 40


# ---------------------------------------------------------------- attention backward
# The pages' setting is training (section "Activation Recompute" reruns each
# layer's forward in the backward pass); the oracle's backward is the exact
# gradient of its forward, pinned here against torch's float64 autograd of
# masked dense attention, central finite differences and invariants.

def _visible(t, row_ids, n_tail, s_k, pool=4):
    """Key positions query t attends: the listed pools' tokens plus up to
    n_tail tokens of its own pool before it."""
    toks = [pool * p + u for p in row_ids if p >= 0 for u in range(pool)]
    start = max((t // pool) * pool, t - n_tail)
    toks += [j for j in range(start, t) if j < s_k]
    return toks


def _torch_grads(x, dout, idx, rows, q_pos0, n_tail, scale):
    """float64 autograd of softmax attention with the visibility mask of each
    listed row; rows that see no key have o = 0 and no gradient."""
    q = x["q"].double()[rows].clone().requires_grad_(True)
    k = x["k"].double().clone().requires_grad_(True)
    v = x["v"].double().clone().requires_grad_(True)
    s_k = k.shape[0]
    mask = torch.zeros(len(rows), s_k, dtype=torch.bool)
    for r, i in enumerate(rows):
        mask[r, _visible(q_pos0 + int(i), idx[r], n_tail, s_k)] = True
    live = mask.any(1)
    lg = torch.einsum("rhd,jd->rhj", q, k) * scale
    lg = lg.masked_fill(~mask[:, None, :], float("-inf"))
    lg = torch.where(live[:, None, None], lg, torch.zeros_like(lg))
    o = torch.softmax(lg, dim=-1) @ v
    o = torch.where(live[:, None, None], o, torch.zeros_like(o))
    (o * dout.double()[rows]).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def _random_idx(rng, rows, q_pos0, n_pools, k_pools):
    idx = np.full((len(rows), k_pools), -1, dtype=np.int32)
    for r, i in enumerate(rows):
        n = min((q_pos0 + int(i)) // 4, n_pools)
        m = min(n, k_pools)
        idx[r, :m] = np.sort(rng.choice(n, size=m, replace=False))
    return idx


@pytest.mark.parametrize("n_tail", [0, 3])
def test_attention_backward_with_every_pool_equals_dense_autograd(n_tail):
    # k >= P: the selection is every earlier pool, so T(t) is dense causal
    # attention (strictly before t with n_tail = 3)
    wl, x = _attn_case(61, h=3, d=32, dv=24, seed=11)
    dout = inputs.make_dout(wl, seed=11)
    P = wl.n_pools
    rows = np.arange(wl.s_q)
    idx = np.full((len(rows), P), -1, dtype=np.int32)
    for r in rows:
        idx[r, :min(r // 4, P)] = np.arange(min(r // 4, P))
    scale = 0.2
    g = oracle.sparse_attn_bwd(x["q"], x["k"], x["v"], idx, dout, P, rows=rows, n_tail=n_tail,
                               scale=scale)
    dq, dk, dv = _torch_grads(x, dout, idx, rows, 0, n_tail, scale)
    np.testing.assert_allclose(g["dq"], dq, rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dk"], dk, rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dv"], dv, rtol=0, atol=1e-11)
    assert np.abs(dk).max() > 0.1 and np.abs(dq).max() > 0.1


@pytest.mark.parametrize("n_tail,q_pos0", [(0, 0), (2, 13), (1, 40)])
def test_attention_backward_sparse_selection_matches_autograd(n_tail, q_pos0):
    wl, x = _attn_case(97, h=2, d=16, dv=40, q_pos0=q_pos0, seed=12 + q_pos0)
    dout = inputs.make_dout(wl, seed=5)
    rng = np.random.default_rng(q_pos0)
    rows = np.arange(wl.s_q)
    idx = _random_idx(rng, rows, q_pos0, wl.n_pools, 5)
    g = oracle.sparse_attn_bwd(x["q"], x["k"], x["v"], idx, dout, 5, q_pos0=q_pos0, rows=rows,
                               n_tail=n_tail, scale=0.3)
    dq, dk, dv = _torch_grads(x, dout, idx, rows, q_pos0, n_tail, 0.3)
    np.testing.assert_allclose(g["dq"], dq, rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dk"], dk, rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dv"], dv, rtol=0, atol=1e-11)


def test_attention_backward_central_differences():
    # the gradient of L = sum dout . o against the function's own values,
    # o evaluated in float64 by a direct softmax over the visible keys
    wl, x = _attn_case(24, h=2, d=8, dv=6, seed=13)
    dout = inputs.make_dout(wl, seed=13)
    rows = np.array([9, 14, 23])
    idx = np.array([[0, -1], [0, 2], [1, 4]], dtype=np.int32)
    scale, n_tail = 0.5, 3
    g = oracle.sparse_attn_bwd(x["q"], x["k"], x["v"], idx, dout, 2, rows=rows, n_tail=n_tail,
                               scale=scale)
    q0, k0, v0 = (x[n].double().numpy() for n in ("q", "k", "v"))
    do = dout.double().numpy()

    def loss(q, k, v):
        tot = 0.0
        for r, i in enumerate(rows):
            toks = _visible(int(i), idx[r], n_tail, k.shape[0])
            for hh in range(q.shape[1]):
                lg = scale * (k[toks] @ q[i, hh])
                p = np.exp(lg - lg.max())
                tot += do[i, hh] @ (p @ v[toks] / p.sum())
        return tot

    eps = 1e-6
    rng = np.random.default_rng(0)
    for name, arr, grad, sel in (
            ("q", q0, g["dq"], None), ("k", k0, g["dk"], None), ("v", v0, g["dv"], None)):
        for _ in range(12):
            if name == "q":
                r = int(rng.integers(len(rows)))
                pos = (int(rows[r]), int(rng.integers(2)), int(rng.integers(8)))
                gpos = (r,) + pos[1:]
            else:
                j = int(rng.choice(_visible(int(rows[-1]), idx[-1], n_tail, 24)))
                pos = (j, int(rng.integers(arr.shape[1])))
                gpos = pos
            hi, lo = arr.copy(), arr.copy()
            hi[pos] += eps
            lo[pos] -= eps
            args_hi = {"q": (hi, k0, v0), "k": (q0, hi, v0), "v": (q0, k0, hi)}[name]
            args_lo = {"q": (lo, k0, v0), "k": (q0, lo, v0), "v": (q0, k0, lo)}[name]
            fd = (loss(*args_hi) - loss(*args_lo)) / (2 * eps)
            assert abs(fd - grad[gpos]) <= 1e-7 * max(1.0, abs(fd)), (name, pos, fd, grad[gpos])


def test_attention_backward_invariants():
    wl, x = _attn_case(130, h=4, d=32, dv=32, seed=14)
    dout = inputs.make_dout(wl, seed=14)
    rng = np.random.default_rng(3)
    rows = np.arange(wl.s_q)
    idx = _random_idx(rng, rows, 0, wl.n_pools, 6)
    g = oracle.sparse_attn_bwd(x["q"], x["k"], x["v"], idx, dout, 6, rows=rows, n_tail=3,
                               scale=0.25, magnitudes=True)
    do = dout.double().numpy()
    # the softmax weights of each (row, head) sum to 1: sum_j dv[j] = sum of dout
    # over the rows that see any key (row 0 sees none)
    np.testing.assert_allclose(g["dv"].sum(0), do[1:].sum((0, 1)), rtol=0, atol=1e-10)
    # sum_j dS_j = 0 for every (row, head): the key gradients sum to zero
    np.testing.assert_allclose(g["dk"].sum(0), 0.0, rtol=0, atol=1e-10)
    # row 0 sees nothing: no query gradient
    assert np.all(g["dq"][0] == 0)
    # the magnitudes bound the values
    for n in ("dq", "dk", "dv"):
        assert np.all(np.abs(g[n]) <= g[n + "_mag"] * (1 + 1e-12) + 1e-300)
    assert g["dq_mag"].max() > 0 and g["dk_mag"].max() > 0


def test_attention_backward_single_key_closed_form():
    # one visible key: the softmax weight is 1 whatever the logit, so dq = 0,
    # dk = 0, and dv of that key is the sum of dout over the heads
    wl, x = _attn_case(16, h=3, d=8, dv=8, seed=15)
    dout = inputs.make_dout(wl, seed=15)
    rows = [1, 5]                         # t = 1: tail {0}; t = 5: tail {4}
    idx = np.full((2, 1), -1, dtype=np.int32)
    g = oracle.sparse_attn_bwd(x["q"], x["k"], x["v"], idx, dout, 1, rows=rows, n_tail=1,
                               scale=0.5)
    do = dout.double().numpy()
    assert np.all(g["dq"] == 0) and np.all(g["dk"] == 0)
    np.testing.assert_allclose(g["dv"][0], do[1].sum(0), rtol=1e-15)
    np.testing.assert_allclose(g["dv"][4], do[5].sum(0), rtol=1e-15)
    assert np.all(g["dv"][[1, 2, 3] + list(range(5, 16))] == 0)


def test_attention_backward_listed_rows_equal_zero_dout_elsewhere():
    wl, x = _attn_case(80, h=2, d=16, seed=16)
    dout = inputs.make_dout(wl, seed=16)
    rng = np.random.default_rng(4)
    rows = np.arange(wl.s_q)
    idx = _random_idx(rng, rows, 0, wl.n_pools, 4)
    pick = np.array([7, 30, 31, 79])
    part = oracle.sparse_attn_bwd(x["q"], x["k"], x["v"], idx[pick], dout, 4, rows=pick,
                                  n_tail=2)
    d0 = torch.zeros_like(dout)
    d0[pick] = dout[pick]
    full = oracle.sparse_attn_bwd(x["q"], x["k"], x["v"], idx, d0, 4, rows=rows, n_tail=2)
    np.testing.assert_array_equal(part["dq"], full["dq"][pick])
    np.testing.assert_array_equal(part["dk"], full["dk"])
    np.testing.assert_array_equal(part["dv"], full["dv"])
    assert np.all(full["dq"][np.setdiff1d(rows, pick)] == 0)


def test_attention_backward_rejects_malformed_rows():
    wl, x = _attn_case(64, seed=17)
    dout = inputs.make_dout(wl, seed=17)
    for bad in ([3, 1, -1, -1], [0, 0, -1, -1], [0, 15, -1, -1]):
        with pytest.raises(RuntimeError):
            oracle.sparse_attn_bwd(x["q"], x["k"], x["v"], np.array([bad], dtype=np.int32),
                                   dout, 4, rows=[60])


# ---------------------------------------------------------------- page figures
# tests/golden/page_figures.txt holds the figures the blog prints, with their
# sections; these tests tie the oracle's shapes to them.

def _page_figures():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "page_figures.txt")
    out = {}
    with open(path) as fh:
        for ln in fh:
            if not ln.strip() or ln.lstrip().startswith("#"):
                continue
            name, size, value = ln.split()[:3]
            out.setdefault(name, {})[size] = int(value)
    return out


def test_page_figures_memory_model_and_selection_size():
    fig = _page_figures()
    # the unchunked per-head score buffer: 2 copies x 4 B x S x S/4 pools x 32 heads
    for size, value in fig["unchunked_indexer_bytes"].items():
        s = int(size)
        assert 2 * 4 * s * (s // fig["pool_size"]["-"]) * 32 == value
    # 512 pools of 4 tokens are the 2048 attended tokens
    assert 512 * fig["pool_size"]["-"] == fig["selected_tokens"]["-"]


def test_page_figures_keys_per_query_from_the_oracle():
    # With all logits 0 (q = 0) the softmax is uniform over the token set, so
    # exp(lse) counts the keys a query attends: 512 pools of 4 plus the 3
    # earlier tokens of its own pool (reading R6) make the page's 2,051.
    fig = _page_figures()
    k_pools = fig["selected_tokens"]["-"] // fig["pool_size"]["-"]
    t = 4 * 1200 + 3                      # t mod 4 = 3: three earlier tokens in its pool
    s_k = t + 1
    q = torch.zeros(1, 2, 64, dtype=torch.bfloat16)
    k = torch.randn(s_k, 64).to(torch.bfloat16)
    v = torch.randn(s_k, 64).to(torch.bfloat16)
    ids = np.arange(0, 2 * k_pools, 2, dtype=np.int32)[None, :]   # 512 pools, all before t
    _, lse = oracle.sparse_attn(q, k, v, ids, k_pools, q_pos0=t, rows=np.array([0]), n_tail=3)
    assert np.allclose(np.exp(lse), fig["keys_per_query"]["-"], rtol=1e-12)
    # the chunk buffer cap the ABI enforces is the page's
    assert fig["chunk_buffer_cap_bytes"]["-"] == 2 ** 31


def test_index_row_validator_accepts_oracle_rows_and_catches_planted_mistakes():
    # the host-side check the GPU tests run on every id row before attention:
    # the oracle's rows pass, and each kind of malformed row is caught
    import parity
    wl = inputs.custom("validator", s_q=90, s_k=90, h_idx=4, d_idx=64, k_pools=6, number=910)
    x = inputs.make_inputs(wl, attention=False)
    idx, _ = oracle.index_topk(x["q_idx"], x["k_idx"], x["w"], wl.k_pools)
    pos = np.arange(wl.s_q)
    parity.validate_index_rows(idx, pos, wl.n_pools, wl.k_pools)
    t = 80  # n(t) = 20 > k
    for plant in ("order", "causal", "pad", "duplicate", "short"):
        bad = idx.copy()
        if plant == "order":
            bad[t, [0, 1]] = bad[t, [1, 0]]
        elif plant == "causal":
            bad[t, -1] = t // 4          # the pool holding t itself
        elif plant == "pad":
            bad[10, -1] = 0              # n(10) = 2: entries 2.. must be -1
        elif plant == "duplicate":
            bad[t, 1] = bad[t, 0]
        else:
            bad[t, -1] = -1              # fewer than min(n, k) ids
        with pytest.raises(AssertionError):
            parity.validate_index_rows(bad, pos, wl.n_pools, wl.k_pools)
