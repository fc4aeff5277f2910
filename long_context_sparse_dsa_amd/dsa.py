"""Python binding of libdsa (argument marshalling only).

Each function has the name of the C entry point it calls (declared in
``include/dsa.h``), takes torch tensors on the current HIP device, passes
their pointers and sizes, and raises ``DsaError`` when the library returns a
non-zero status.  All computation happens in the library's HIP kernels; there
is no other implementation behind these names.  If ``libdsa.so`` has not been
built, the first call raises instead of running anything else.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
DSA_BF16, DSA_FP8_E4M3 = 0, 1
STATUS_NAMES = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED",
                3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_HIP"}


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


_lock = threading.Lock()
_lib = None

_i64, _int, _vp, _f = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdsa.so (once).  Raises FileNotFoundError if it is not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"{path} is missing: build it with long_context_sparse_dsa_amd/build.py")
        lib = ctypes.CDLL(path)
        lib.dsa_version.restype = _int
        lib.dsa_version.argtypes = []
        lib.dsa_last_error.restype = ctypes.c_char_p
        lib.dsa_last_error.argtypes = []
        lib.dsa_index_workspace_size.restype = _int
        lib.dsa_index_workspace_size.argtypes = [
            _i64, _i64, _int, _int, _int, _int, _i64, _int, ctypes.POINTER(ctypes.c_size_t),
            ctypes.POINTER(_i64)]
        lib.dsa_index_score_topk.restype = _int
        lib.dsa_index_score_topk.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _int, _int, _int, _i64, _int,
            _vp, _vp, _vp, ctypes.c_size_t, _vp]
        lib.dsa_index_score_topk_noalloc.restype = _int
        lib.dsa_index_score_topk_noalloc.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _int, _int, _int, _i64, _int,
            _vp, _vp, _vp]
        lib.dsa_index_score_topk_gated.restype = _int
        lib.dsa_index_score_topk_gated.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _int, _int, _int, _i64,
            _int, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        lib.dsa_index_scores_workspace_size.restype = _int
        lib.dsa_index_scores_workspace_size.argtypes = [
            _i64, _i64, _int, _int, _int, _int, _i64, ctypes.POINTER(ctypes.c_size_t)]
        lib.dsa_index_scores.restype = _int
        lib.dsa_index_scores.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _int, _int, _int, _i64, _i64,
            _vp, _vp, ctypes.c_size_t, _vp]
        lib.dsa_index_scores_gated.restype = _int
        lib.dsa_index_scores_gated.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _int, _int, _int, _i64,
            _i64, _vp, _vp, ctypes.c_size_t, _vp]
        lib.dsa_sparse_attn_fwd.restype = _int
        lib.dsa_sparse_attn_fwd.argtypes = [
            _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _int, _int, _int, _f, _vp,
            _vp, _vp]
        lib.dsa_sparse_attn_bwd_workspace_size.restype = _int
        lib.dsa_sparse_attn_bwd_workspace_size.argtypes = [
            _i64, _i64, _int, _i64, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(_i64)]
        lib.dsa_sparse_attn_bwd.restype = _int
        lib.dsa_sparse_attn_bwd.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _int, _int,
            _int, ctypes.c_float, _i64, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        lib.dsa_profile_enable.restype = _int
        lib.dsa_profile_enable.argtypes = [_int]
        lib.dsa_profile_read.restype = _int
        lib.dsa_profile_read.argtypes = [ctypes.POINTER(KernelStat), _int, ctypes.POINTER(_int)]
        _lib = lib
        return lib


def _check(status: int):
    if status != DSA_OK:
        raise DsaError(status, _lib.dsa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(cond: bool, what: str):
    if not cond:
        raise ValueError(what)


def dsa_version() -> int:
    return load_library().dsa_version()


def dsa_index_workspace_size(s_q: int, s_k: int, h_idx: int, d_idx: int, k_pools: int,
                             pool_size: int = 4, chunk_q: int = 0,
                             dtype: int = DSA_BF16) -> tuple[int, int]:
    """(workspace bytes, chunk_q used)."""
    lib = load_library()
    nbytes = ctypes.c_size_t(0)
    cq = _i64(0)
    _check(lib.dsa_index_workspace_size(s_q, s_k, h_idx, d_idx, k_pools, pool_size, chunk_q,
                                        dtype, ctypes.byref(nbytes), ctypes.byref(cq)))
    return nbytes.value, cq.value


def _indexer_shapes(q_idx, k_idx, w):
    _need(q_idx.dim() == 3 and k_idx.dim() == 2, "q_idx must be [S_q,H_I,D_I], k_idx [S_k,D_I]")
    s_q, h_idx, d_idx = q_idx.shape
    s_k = k_idx.shape[0]
    _need(k_idx.shape[1] == d_idx, "k_idx dim must match q_idx")
    _need(q_idx.is_contiguous() and k_idx.is_contiguous(), "q_idx and k_idx must be contiguous")
    _need(w.dtype == torch.float32, "w must be fp32")
    if w.dim() == 1:
        _need(w.shape[0] == h_idx, "w must be [H_I] or [S_q, H_I]")
        w_stride = 0
    else:
        _need(w.dim() == 2 and w.shape[0] == s_q and w.shape[1] == h_idx and w.stride(1) == 1,
              "w must be [H_I] or [S_q, H_I] with unit inner stride")
        w_stride = w.stride(0)
    if q_idx.dtype == torch.bfloat16:
        _need(k_idx.dtype == torch.bfloat16, "q_idx and k_idx must share a dtype")
        dtype = DSA_BF16
    elif q_idx.dtype == torch.float8_e4m3fn:
        _need(k_idx.dtype == torch.float8_e4m3fn, "q_idx and k_idx must share a dtype")
        dtype = DSA_FP8_E4M3
    else:
        raise ValueError("q_idx must be bfloat16 or float8_e4m3fn")
    return s_q, s_k, h_idx, d_idx, w_stride, dtype


def dsa_index_scores_workspace_size(s_q: int, s_k: int, h_idx: int, d_idx: int,
                                    n_rows: int, pool_size: int = 4,
                                    dtype: int = DSA_BF16) -> int:
    lib = load_library()
    nbytes = ctypes.c_size_t(0)
    _check(lib.dsa_index_scores_workspace_size(s_q, s_k, h_idx, d_idx, pool_size, dtype, n_rows,
                                               ctypes.byref(nbytes)))
    return nbytes.value


def new_workspace(nbytes: int, device=None) -> torch.Tensor:
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device or "cuda")


def _gate_ptr(k_gate, k_idx):
    if k_gate is None:
        return None
    _need(k_gate.dtype == torch.float32 and k_gate.dim() == 1 and k_gate.is_contiguous()
          and k_gate.shape[0] == k_idx.shape[0], "k_gate must be contiguous fp32 [S_k]")
    return _ptr(k_gate)


def _score_topk(fn, q_idx, k_idx, k_gate, w, k_pools, q_pos0, chunk_q, q_scale, k_scale,
                idx_out, score_out, want_scores, workspace, stream):
    lib = load_library()
    s_q, s_k, h_idx, d_idx, w_stride, dtype = _indexer_shapes(q_idx, k_idx, w)
    dev = q_idx.device
    nbytes, _ = dsa_index_workspace_size(s_q, s_k, h_idx, d_idx, k_pools, 4, chunk_q, dtype)
    if workspace is None:
        workspace = new_workspace(nbytes, dev)
    if idx_out is None:
        idx_out = torch.empty((s_q, k_pools), dtype=torch.int32, device=dev)
    if score_out is None and want_scores:
        score_out = torch.empty((s_q, k_pools), dtype=torch.float32, device=dev)
    gate = [] if fn == "dsa_index_score_topk" else [_gate_ptr(k_gate, k_idx)]
    _check(getattr(lib, fn)(
        _ptr(q_idx), _ptr(k_idx), *gate, _ptr(q_scale), _ptr(k_scale), _ptr(w), w_stride, s_q,
        s_k, q_pos0, h_idx, d_idx, 4, k_pools, chunk_q, dtype, _ptr(idx_out), _ptr(score_out),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return idx_out, score_out


def dsa_index_score_topk(q_idx: torch.Tensor, k_idx: torch.Tensor, w: torch.Tensor,
                         k_pools: int, *, q_pos0: int = 0, chunk_q: int = 0,
                         q_scale: torch.Tensor | None = None,
                         k_scale: torch.Tensor | None = None,
                         idx_out: torch.Tensor | None = None,
                         score_out: torch.Tensor | None = None,
                         want_scores: bool = False,
                         workspace: torch.Tensor | None = None, stream=None):
    """Pool (mean of 4 keys), score in chunks and keep the top ``k_pools``
    pools per query.

    Returns (idx [S_q, k_pools] int32, scores [S_q, k_pools] fp32 or None)."""
    return _score_topk("dsa_index_score_topk", q_idx, k_idx, None, w, k_pools, q_pos0, chunk_q,
                       q_scale, k_scale, idx_out, score_out, want_scores, workspace, stream)


def dsa_index_score_topk_noalloc(q_idx: torch.Tensor, k_idx: torch.Tensor, w: torch.Tensor,
                                 k_pools: int, *, q_pos0: int = 0, chunk_q: int = 0,
                                 q_scale: torch.Tensor | None = None,
                                 k_scale: torch.Tensor | None = None,
                                 idx_out: torch.Tensor | None = None,
                                 score_out: torch.Tensor | None = None,
                                 want_scores: bool = False, stream=None):
    """dsa_index_score_topk without a workspace: the library uses its own
    per-GPU scratch array and allocates nothing.  Outputs not passed in are
    allocated here, by the caller's side of the boundary.

    Returns (idx [S_q, k_pools] int32, scores [S_q, k_pools] fp32 or None)."""
    lib = load_library()
    s_q, s_k, h_idx, d_idx, w_stride, dtype = _indexer_shapes(q_idx, k_idx, w)
    dev = q_idx.device
    if idx_out is None:
        idx_out = torch.empty((s_q, k_pools), dtype=torch.int32, device=dev)
    if score_out is None and want_scores:
        score_out = torch.empty((s_q, k_pools), dtype=torch.float32, device=dev)
    _check(lib.dsa_index_score_topk_noalloc(
        _ptr(q_idx), _ptr(k_idx), _ptr(q_scale), _ptr(k_scale), _ptr(w), w_stride, s_q, s_k,
        q_pos0, h_idx, d_idx, 4, k_pools, chunk_q, dtype, _ptr(idx_out), _ptr(score_out),
        _stream(stream)))
    return idx_out, score_out


def dsa_index_score_topk_gated(q_idx: torch.Tensor, k_idx: torch.Tensor, k_gate: torch.Tensor,
                               w: torch.Tensor, k_pools: int, *, q_pos0: int = 0,
                               chunk_q: int = 0, q_scale: torch.Tensor | None = None,
                               k_scale: torch.Tensor | None = None,
                               idx_out: torch.Tensor | None = None,
                               score_out: torch.Tensor | None = None,
                               want_scores: bool = False,
                               workspace: torch.Tensor | None = None, stream=None):
    """As dsa_index_score_topk, with each pooled key the gate-weighted sum of
    its 4 keys (k_gate: per-token gates [S_k] fp32)."""
    return _score_topk("dsa_index_score_topk_gated", q_idx, k_idx, k_gate, w, k_pools, q_pos0,
                       chunk_q, q_scale, k_scale, idx_out, score_out, want_scores, workspace,
                       stream)


def _scores(fn, q_idx, k_idx, k_gate, w, row0, n_rows, q_pos0, q_scale, k_scale, workspace,
            stream):
    lib = load_library()
    s_q, s_k, h_idx, d_idx, w_stride, dtype = _indexer_shapes(q_idx, k_idx, w)
    n_rows = s_q - row0 if n_rows is None else n_rows
    dev = q_idx.device
    n_pools = s_k // 4
    need = dsa_index_scores_workspace_size(s_q, s_k, h_idx, d_idx, n_rows, 4, dtype)
    if workspace is None:
        workspace = new_workspace(need, dev)
    out = torch.empty((n_rows, n_pools), dtype=torch.float32, device=dev)
    gate = [] if fn == "dsa_index_scores" else [_gate_ptr(k_gate, k_idx)]
    _check(getattr(lib, fn)(
        _ptr(q_idx), _ptr(k_idx), *gate, _ptr(q_scale), _ptr(k_scale), _ptr(w), w_stride, s_q,
        s_k, q_pos0, h_idx, d_idx, 4, dtype, row0, n_rows, _ptr(out), _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return out


def dsa_index_scores(q_idx: torch.Tensor, k_idx: torch.Tensor, w: torch.Tensor, *,
                     row0: int = 0, n_rows: int | None = None, q_pos0: int = 0,
                     q_scale: torch.Tensor | None = None, k_scale: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Dense fp32 scores [n_rows, P] of rows [row0, row0+n_rows); -inf = not eligible."""
    return _scores("dsa_index_scores", q_idx, k_idx, None, w, row0, n_rows, q_pos0, q_scale,
                   k_scale, workspace, stream)


def dsa_index_scores_gated(q_idx: torch.Tensor, k_idx: torch.Tensor, k_gate: torch.Tensor,
                           w: torch.Tensor, *, row0: int = 0, n_rows: int | None = None,
                           q_pos0: int = 0, q_scale: torch.Tensor | None = None,
                           k_scale: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """As dsa_index_scores, with gate-weighted pooled keys (k_gate [S_k] fp32)."""
    return _scores("dsa_index_scores_gated", q_idx, k_idx, k_gate, w, row0, n_rows, q_pos0,
                   q_scale, k_scale, workspace, stream)


def dsa_sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, *,
                        q_pos0: int = 0, n_tail: int = 0, softmax_scale: float = 0.0,
                        out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                        want_lse: bool = False, stream=None):
    """Attention over the kept pools.  Returns (out [S_q,H,Dv] bf16, lse [S_q,H] or None)."""
    lib = load_library()
    _need(q.dim() == 3 and k.dim() == 2 and v.dim() == 2 and idx.dim() == 2,
          "q [S_q,H,D], k [S_k,D], v [S_k,Dv], idx [S_q,k_pools]")
    _need(q.dtype == k.dtype == v.dtype == torch.bfloat16, "q, k, v must be bfloat16")
    _need(idx.dtype == torch.int32, "idx must be int32")
    _need(all(t.is_contiguous() for t in (q, k, v, idx)), "inputs must be contiguous")
    s_q, h, d = q.shape
    s_k, dv = v.shape
    _need(k.shape == (s_k, d), "k must be [S_k, D]")
    _need(idx.shape[0] == s_q, "idx must have one row per query")
    k_pools = idx.shape[1]
    if out is None:
        out = torch.empty((s_q, h, dv), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((s_q, h), dtype=torch.float32, device=q.device)
    _check(lib.dsa_sparse_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(idx), s_q, s_k, q_pos0, h, d, dv, k_pools, 4, n_tail,
        float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def dsa_sparse_attn_bwd_workspace_size(s_q: int, s_k: int, h: int, chunk_q: int = 0):
    """(bytes, chunk_q used) of the backward's workspace."""
    nb = ctypes.c_size_t(0)
    cq = _i64(0)
    _check(load_library().dsa_sparse_attn_bwd_workspace_size(s_q, s_k, h, chunk_q,
                                                              ctypes.byref(nb), ctypes.byref(cq)))
    return nb.value, cq.value


def dsa_sparse_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                        out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor, *,
                        q_pos0: int = 0, n_tail: int = 0, softmax_scale: float = 0.0,
                        chunk_q: int = 0, dq: torch.Tensor | None = None,
                        dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stream=None):
    """Gradients of the attention over the kept pools for the upstream
    gradient dout.  Returns (dq [S_q,H,D], dk [S_k,D], dv [S_k,Dv]), fp32."""
    lib = load_library()
    _need(q.dim() == 3 and k.dim() == 2 and v.dim() == 2 and idx.dim() == 2,
          "q [S_q,H,D], k [S_k,D], v [S_k,Dv], idx [S_q,k_pools]")
    _need(q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype == torch.bfloat16,
          "q, k, v, out, dout must be bfloat16")
    _need(idx.dtype == torch.int32 and lse.dtype == torch.float32, "idx int32, lse fp32")
    _need(all(t.is_contiguous() for t in (q, k, v, idx, out, dout, lse)),
          "inputs must be contiguous")
    s_q, h, d = q.shape
    s_k, dvd = v.shape
    _need(k.shape == (s_k, d), "k must be [S_k, D]")
    _need(idx.shape[0] == s_q, "idx must have one row per query")
    _need(out.shape == (s_q, h, dvd) and dout.shape == out.shape, "out, dout [S_q, H, Dv]")
    _need(lse.shape == (s_q, h), "lse [S_q, H]")
    k_pools = idx.shape[1]
    dev = q.device
    if dq is None:
        dq = torch.empty((s_q, h, d), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty((s_k, d), dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty((s_k, dvd), dtype=torch.float32, device=dev)
    nbytes, _ = dsa_sparse_attn_bwd_workspace_size(s_q, s_k, h, chunk_q)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.dsa_sparse_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(out), _ptr(dout), _ptr(lse), s_q, s_k,
        q_pos0, h, d, dvd, k_pools, 4, n_tail, float(softmax_scale), chunk_q, _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(workspace), workspace.numel(), _stream(stream)))
    return dq, dk, dv


def dsa_profile_enable(on: bool = True):
    _check(load_library().dsa_profile_enable(1 if on else 0))


def dsa_profile_read() -> dict:
    """{kernel kind: (launches, total_ms)} since the last read."""
    lib = load_library()
    arr = (KernelStat * 16)()
    n = _int(0)
    _check(lib.dsa_profile_read(arr, 16, ctypes.byref(n)))
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n.value)}
