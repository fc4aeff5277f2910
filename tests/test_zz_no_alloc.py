"""dsa_index_score_topk_noalloc (no workspace argument, the library's own
per-GPU scratch array) against dsa_index_score_topk with a caller workspace:
ids and kept scores bit-identical, on calls in a row whose inputs shrink and
change shape, so that what one call leaves in the shared scratch array cannot
reach the next call's results."""
import math
import sys

import numpy as np
import pytest
import torch

from long_context_sparse_dsa_amd import dsa, inputs
import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.load_library()


def _compare(wl, fp8=False, w_per_query=False, scales=(1.0, 1.0)):
    print(f"[no-alloc] {wl.name} s_q={wl.s_q} s_k={wl.s_k} q_pos0={wl.q_pos0} "
          f"H_I={wl.h_idx} D_I={wl.d_idx} k={wl.k_pools} fp8={fp8}", flush=True)
    x = inputs.make_inputs(wl, attention=False, w_per_query=w_per_query)
    dev = torch.device("cuda")
    qn, kn = ("q_idx8", "k_idx8") if fp8 else ("q_idx", "k_idx")
    q_idx, k_idx, w = x[qn].to(dev), x[kn].to(dev), x["w"].to(dev)
    kw = {}
    if fp8:
        kw = dict(q_scale=torch.tensor([scales[0]], dtype=torch.float32, device=dev),
                  k_scale=torch.tensor([scales[1]], dtype=torch.float32, device=dev))
    idx_a, sc_a = dsa.dsa_index_score_topk(q_idx, k_idx, w, wl.k_pools, q_pos0=wl.q_pos0,
                                           want_scores=True, **kw)
    idx_b, sc_b = dsa.dsa_index_score_topk_noalloc(q_idx, k_idx, w, wl.k_pools,
                                                   q_pos0=wl.q_pos0, want_scores=True, **kw)
    idx_c, _ = dsa.dsa_index_score_topk_noalloc(q_idx, k_idx, w, wl.k_pools, q_pos0=wl.q_pos0,
                                                **kw)
    torch.cuda.synchronize()
    assert torch.equal(idx_a, idx_b), "ids differ from the workspace entry point's"
    assert torch.equal(idx_a, idx_c), "ids without score_out differ"
    assert torch.equal(sc_a.view(torch.int32), sc_b.view(torch.int32)), "kept scores differ"
    parity.validate_index_rows(idx_b.cpu().numpy(), wl.q_pos0 + np.arange(wl.s_q), wl.n_pools,
                               wl.k_pools)


def test_noalloc_matches_the_workspace_entry_point_on_calls_in_a_row():
    # 1: long rows (31K-32K pools, bounded scoring and rescoring); the
    # scratch holds 1728-query chunks here, the workspace call one chunk of
    # 6016, so the chunking differs as well
    _compare(inputs.custom("noalloc_long", s_q=6000, s_k=131072, q_pos0=125072, h_idx=32,
                           d_idx=128, k_pools=512, idx_std=1 / math.sqrt(128), number=480))
    # 2: smaller, fp8 indexer (another workspace layout over the same scratch)
    _compare(inputs.custom("noalloc_fp8", s_q=2100, s_k=2100, h_idx=32, d_idx=96, k_pools=48,
                           fp8=True, number=481), fp8=True, scales=(0.5, -2.0))
    # 3: smaller still, bf16, other head count and width, per-query weights,
    # offset queries
    _compare(inputs.custom("noalloc_small", s_q=700, s_k=3003, q_pos0=2303, h_idx=16,
                           d_idx=96, k_pools=100, idx_std=0.1, number=482), w_per_query=True)


def test_noalloc_rejects_what_does_not_fit_before_launching():
    dev = torch.device("cuda")
    wl = inputs.custom("noalloc_reject", s_q=64, s_k=131072, h_idx=32, d_idx=128, k_pools=512)
    q = torch.zeros((wl.s_q, 32, 128), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((wl.s_k, 128), dtype=torch.bfloat16, device=dev)
    w = torch.ones(32, dtype=torch.float32, device=dev)
    idx = torch.full((wl.s_q, wl.k_pools), 7, dtype=torch.int32, device=dev)
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_index_score_topk_noalloc(q, k, w, wl.k_pools, chunk_q=8192, idx_out=idx)
    assert e.value.status == dsa.DSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((idx == 7).all()), "a rejected call wrote its output"
