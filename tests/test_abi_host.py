"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point the header declares, sizes workspaces, and rejects bad
arguments with a status code before touching the device."""
import ctypes
import os
import re

import pytest

from long_context_sparse_dsa_amd import dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa.LIB_PATH):
        pytest.skip("libdsa.so not built")
    return dsa.load_library()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("dsa_index_score_topk", "dsa_sparse_attn_fwd", "dsa_index_workspace_size",
              "dsa_index_scores", "dsa_index_scores_workspace_size", "dsa_last_error",
              "dsa_version", "dsa_profile_enable", "dsa_profile_read"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.dsa_version() == 100


def test_workspace_size_matches_layout(lib):
    # 128k tokens, 32x128 indexer, chunks of 256: pooled table 32768 x 256 x 2 B
    # plus 256 x 32768 fp32 scores -- the page keeps each chunk under 2 GiB
    nbytes, cq = dsa.dsa_index_workspace_size(131072, 131072, 32, 128, 512, 4, 256)
    assert cq == 256
    # hi bf16 + lo E4M3 + lo scales + per-pool bound factors (2 x fp32), the
    # chunk's packed query tiles (one query per tile at 32 heads, three spare;
    # 12288 query bytes + 224 bytes of weights, scales and bound factors,
    # rounded to 128), per-query bound factors (2 x fp32), the scores
    assert nbytes == (32768 * 128 * 2 + 32768 * 128 + 32768 + 32768 * 8
                      + (256 + 3) * 12544 + 256 * 8 + 256 * 32768 * 4)
    assert 256 * 32768 * 4 <= 2 ** 31
    # default chunk
    _, cq = dsa.dsa_index_workspace_size(32768, 32768, 32, 128, 512)
    assert cq > 0 and cq % 64 == 0


def test_chunk_buffer_cap_enforced(lib):
    # one GPU's share of 1M tokens: 262144 pools; 2048 rows x 1 MiB = 2 GiB is the cap
    nbytes, _ = dsa.dsa_index_workspace_size(131072, 1 << 20, 32, 128, 512, 4, 2048)
    assert nbytes >= 2048 * 262144 * 4
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_index_workspace_size(131072, 1 << 20, 32, 128, 512, 4, 2112)
    assert e.value.status == dsa.DSA_ERR_UNSUPPORTED


@pytest.mark.parametrize("args,status", [
    (dict(h_idx=12), dsa.DSA_ERR_UNSUPPORTED),
    (dict(d_idx=80), dsa.DSA_ERR_UNSUPPORTED),
    (dict(k_pools=0), dsa.DSA_ERR_UNSUPPORTED),
    (dict(k_pools=4096), dsa.DSA_ERR_UNSUPPORTED),
    (dict(pool_size=8), dsa.DSA_ERR_UNSUPPORTED),
    (dict(chunk_q=100), dsa.DSA_ERR_UNSUPPORTED),
    (dict(chunk_q=-64), dsa.DSA_ERR_INVALID_ARG),
    (dict(s_q=-1), dsa.DSA_ERR_INVALID_ARG),
    (dict(dtype=7), dsa.DSA_ERR_INVALID_ARG),
])
def test_workspace_size_rejects(lib, args, status):
    kw = dict(s_q=1024, s_k=1024, h_idx=32, d_idx=128, k_pools=64, pool_size=4, chunk_q=0,
              dtype=0)
    kw.update(args)
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_index_workspace_size(**kw)
    assert e.value.status == status
    assert lib.dsa_last_error().decode() != ""


def _call_topk(lib, **over):
    a = dict(q_idx=0x1000, k_idx=0x2000, q_scale=None, k_scale=None, w=0x3000, w_stride=0,
             s_q=64, s_k=64, q_pos0=0, h_idx=32, d_idx=128, pool=4, k=8, chunk=0, dtype=0,
             idx=0x4000, score=None, ws=0x5000, ws_bytes=1 << 30, stream=None)
    a.update(over)
    return lib.dsa_index_score_topk(
        a["q_idx"], a["k_idx"], a["q_scale"], a["k_scale"], a["w"], a["w_stride"], a["s_q"],
        a["s_k"], a["q_pos0"], a["h_idx"], a["d_idx"], a["pool"], a["k"], a["chunk"], a["dtype"],
        a["idx"], a["score"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q_idx=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(w=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(idx=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(q_idx=0x1004), dsa.DSA_ERR_INVALID_ARG),          # misaligned
    (dict(w_stride=7), dsa.DSA_ERR_INVALID_ARG),            # 0 < stride < h_idx
    (dict(q_scale=0x6000), dsa.DSA_ERR_INVALID_ARG),        # scales are fp8-only
    (dict(ws=None), dsa.DSA_ERR_WORKSPACE),
    (dict(ws_bytes=1024), dsa.DSA_ERR_WORKSPACE),
    (dict(h_idx=64), dsa.DSA_ERR_UNSUPPORTED),
    (dict(d_idx=192), dsa.DSA_ERR_UNSUPPORTED),
    (dict(s_k=1 << 31), dsa.DSA_ERR_UNSUPPORTED),
])
def test_index_score_topk_rejects_before_launch(lib, over, status):
    # all pointers are fake: a call that got past validation would fault, so
    # these tests also show that nothing is enqueued on a rejected call
    assert _call_topk(lib, **over) == status
    assert lib.dsa_last_error().decode() != ""


def test_empty_query_set_is_a_no_op(lib):
    assert _call_topk(lib, s_q=0, q_idx=None, w=None, idx=None, ws=None, ws_bytes=0) == dsa.DSA_OK


def _call_attn(lib, **over):
    a = dict(q=0x1000, k=0x2000, v=0x3000, idx=0x4000, s_q=16, s_k=64, q_pos0=0, h=16, d=128,
             dv=128, k_pools=8, pool=4, n_tail=0, scale=0.0, out=0x5000, lse=None, stream=None)
    a.update(over)
    return lib.dsa_sparse_attn_fwd(a["q"], a["k"], a["v"], a["idx"], a["s_q"], a["s_k"],
                                   a["q_pos0"], a["h"], a["d"], a["dv"], a["k_pools"], a["pool"],
                                   a["n_tail"], a["scale"], a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(h=17), dsa.DSA_ERR_UNSUPPORTED),
    (dict(h=0), dsa.DSA_ERR_UNSUPPORTED),
    (dict(d=80), dsa.DSA_ERR_UNSUPPORTED),
    (dict(dv=256), dsa.DSA_ERR_UNSUPPORTED),
    (dict(k_pools=0), dsa.DSA_ERR_UNSUPPORTED),
    (dict(n_tail=4), dsa.DSA_ERR_INVALID_ARG),
    (dict(n_tail=-1), dsa.DSA_ERR_INVALID_ARG),
    (dict(pool=2), dsa.DSA_ERR_UNSUPPORTED),
    (dict(q=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(out=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(lse=0x6002), dsa.DSA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), dsa.DSA_ERR_INVALID_ARG),
    (dict(s_q=-3), dsa.DSA_ERR_INVALID_ARG),
])
def test_sparse_attn_rejects_before_launch(lib, over, status):
    assert _call_attn(lib, **over) == status
    assert lib.dsa_last_error().decode() != ""


def test_index_scores_rejects_rows_out_of_range(lib):
    st = lib.dsa_index_scores(0x1000, 0x2000, None, None, 0x3000, 0, 64, 64, 0, 32, 128, 4, 0,
                              60, 8, 0x4000, 0x5000, 1 << 20, None)
    assert st == dsa.DSA_ERR_INVALID_ARG


def test_fp8_scale_pointers(lib):
    # scales are fp8-only device scalars; a misaligned one is rejected
    assert _call_topk(lib, dtype=1, q_scale=0x6002) == dsa.DSA_ERR_INVALID_ARG
    assert _call_topk(lib, dtype=0, k_scale=0x6000) == dsa.DSA_ERR_INVALID_ARG


def test_fp8_workspace_layout(lib):
    # codes P x d_idx, then fp32 scales, each rounded to 256 B, then the buffer
    nbytes, cq = dsa.dsa_index_workspace_size(65536, 65536, 32, 96, 512, 4, 256, dsa.DSA_FP8_E4M3)
    assert cq == 256
    assert nbytes == 16384 * 96 + 16384 * 4 + 256 * 16384 * 4
    assert dsa.dsa_index_scores_workspace_size(65536, 65536, 32, 96, 16, 4,
                                               dsa.DSA_FP8_E4M3) == 16384 * 96 + 16384 * 4
    r = lambda x: (x + 255) // 256 * 256
    # 8 heads: 4 queries per tile, 25 tiles + 3 spare; per-pool and per-query
    # bound factors (2 x fp32) after the scales and after the tiles
    assert dsa.dsa_index_scores_workspace_size(5000, 4000, 8, 128, 100) == (
        r(1000 * 256) + r(1000 * 128) + r(1000) + r(1000 * 8) + r(28 * 12544) + r(100 * 8))
    # rows are scored 4096 at a time: the tiles stop growing there
    assert dsa.dsa_index_scores_workspace_size(8192, 4000, 8, 128, 8192) == (
        r(1000 * 256) + r(1000 * 128) + r(1000) + r(1000 * 8) + r(1027 * 12544) + r(4096 * 8))


def test_gated_entry_points_check_the_gate(lib):
    a = [0x1000, 0x2000]
    rest = [None, None, 0x3000, 0, 64, 64, 0, 32, 128, 4, 8, 0, 0, 0x4000, None, 0x5000, 1 << 30,
            None]
    # a missing or misaligned gate is rejected before anything is launched
    assert lib.dsa_index_score_topk_gated(*a, None, *rest) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_index_score_topk_gated(*a, 0x6004, *rest) == dsa.DSA_ERR_INVALID_ARG
    assert "k_gate" in lib.dsa_last_error().decode()
    st = lib.dsa_index_scores_gated(0x1000, 0x2000, 0x6008, None, None, 0x3000, 0, 64, 64, 0, 32,
                                    128, 4, 0, 0, 8, 0x4000, 0x5000, 1 << 20, None)
    assert st == dsa.DSA_ERR_INVALID_ARG


def test_profile_read_empty(lib):
    assert dsa.dsa_profile_read() == {}


def _call_bwd(lib, **over):
    a = dict(q=0x1000, k=0x2000, v=0x3000, idx=0x4000, out=0x5000, dout=0x6000, lse=0x7000,
             s_q=16, s_k=64, q_pos0=0, h=16, d=128, dv=128, k_pools=8, pool=4, n_tail=0,
             scale=0.0, chunk=0, dq=0x8000, dk=0x9000, dv_grad=0xA000, ws=0xB000,
             ws_bytes=1 << 30, stream=None)
    a.update(over)
    return lib.dsa_sparse_attn_bwd(
        a["q"], a["k"], a["v"], a["idx"], a["out"], a["dout"], a["lse"], a["s_q"], a["s_k"],
        a["q_pos0"], a["h"], a["d"], a["dv"], a["k_pools"], a["pool"], a["n_tail"], a["scale"],
        a["chunk"], a["dq"], a["dk"], a["dv_grad"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(h=17), dsa.DSA_ERR_UNSUPPORTED),
    (dict(d=80), dsa.DSA_ERR_UNSUPPORTED),
    (dict(n_tail=4), dsa.DSA_ERR_INVALID_ARG),
    (dict(lse=None), dsa.DSA_ERR_INVALID_ARG),        # the forward's lse is required
    (dict(dout=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(dk=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(dq=0x8004), dsa.DSA_ERR_INVALID_ARG),       # misaligned
    (dict(chunk=100), dsa.DSA_ERR_UNSUPPORTED),       # not a multiple of 64
    (dict(chunk=-64), dsa.DSA_ERR_INVALID_ARG),
    (dict(ws=None), dsa.DSA_ERR_WORKSPACE),
    (dict(ws_bytes=100), dsa.DSA_ERR_WORKSPACE),
])
def test_sparse_attn_bwd_rejects_before_launch(lib, over, status):
    assert _call_bwd(lib, **over) == status
    assert lib.dsa_last_error().decode() != ""


def test_sparse_attn_bwd_workspace_layout(lib):
    # delta [s_q, h] fp32 rounded to 256 B, then the bitmap: chunk / 32 rows
    # of ceil(s_k / 4) words, rounded up to 4, per chunk, for every chunk
    # when that fits 1 GiB, else for one (rounded to 256 B), then the pool
    # slots' counts and order, one word per slot (the stride) each, rounded
    # to 256 B
    # default chunk: max(1024, min(1536, 3 slots / 32), slots / 32), at most
    # 16384 and s_q (86 chunks of 1536 queries at 128k)
    nbytes, cq = dsa.dsa_sparse_attn_bwd_workspace_size(131072, 131072, 16)
    assert cq == 1536
    assert nbytes == 131072 * 16 * 4 + 86 * (32768 * 48 * 4) + 2 * 32768 * 4
    _, cq = dsa.dsa_sparse_attn_bwd_workspace_size(65536, 65536, 16)
    assert cq == 1536
    _, cq = dsa.dsa_sparse_attn_bwd_workspace_size(32768, 32768, 16)
    assert cq == 1024
    # one GPU's share of 1M keys: every chunk's bitmap would take 4 GiB, so
    # one chunk's (8192 queries)
    nbytes, cq = dsa.dsa_sparse_attn_bwd_workspace_size(131072, 1 << 20, 16)
    assert cq == 8192
    assert nbytes == 131072 * 16 * 4 + 262144 * 256 * 4 + 2 * 262144 * 4
    _, cq = dsa.dsa_sparse_attn_bwd_workspace_size(131072, 1 << 22, 16)
    assert cq == 16384
    _, cq = dsa.dsa_sparse_attn_bwd_workspace_size(1000, 1 << 20, 16)
    assert cq == 1024
    nbytes, cq = dsa.dsa_sparse_attn_bwd_workspace_size(100, 203, 5, 64)
    # 51 slots -> stride 52; two chunks' bitmaps of 2 word rows
    assert cq == 64 and nbytes == 2048 + 1024 + 2 * 256
    nbytes, cq = dsa.dsa_sparse_attn_bwd_workspace_size(100, 203, 5)
    assert cq == 128
    # one GPU's share of 1M keys: 262144 pool rows; 65536 queries per chunk
    # would need a 2 GiB bitmap, which is the cap
    dsa.dsa_sparse_attn_bwd_workspace_size(131072, 1 << 20, 16, 65536)
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_sparse_attn_bwd_workspace_size(131072, (1 << 20) + 4, 16, 65536)
    assert e.value.status == dsa.DSA_ERR_UNSUPPORTED


def test_noalloc_rejects_before_touching_the_device(lib):
    # argument and size checks come before any HIP call, so these run on a
    # host without a GPU; the fake pointers are never dereferenced
    p = ctypes.c_void_p(4096)
    nul = ctypes.c_void_p(None)

    def call(s_q, s_k, chunk_q, q=p, dtype=dsa.DSA_BF16, k_pools=512):
        return lib.dsa_index_score_topk_noalloc(q, p, nul, nul, p, 0, s_q, s_k, 0, 32, 128, 4,
                                                k_pools, chunk_q, dtype, p, nul, nul)

    # pooled keys of 2M tokens do not fit the 256 MiB scratch array
    assert call(64, 1 << 21, 0) == dsa.DSA_ERR_UNSUPPORTED
    assert b"scratch" in lib.dsa_last_error()
    # a chunk whose buffer does not fit it
    assert call(8192, 131072, 8192) == dsa.DSA_ERR_WORKSPACE
    assert call(64, 131072, 100) == dsa.DSA_ERR_UNSUPPORTED        # not a multiple of 64
    assert call(64, 131072, 0, q=nul) == dsa.DSA_ERR_INVALID_ARG  # missing q_idx
    assert call(64, 131072, 0, k_pools=0) == dsa.DSA_ERR_UNSUPPORTED
    assert call(0, 131072, 0) == dsa.DSA_OK                        # no query: nothing to do
