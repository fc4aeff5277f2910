"""ctypes binding to the plain CPU oracle in ``dsa_oracle.c``.

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the package smoke
check and by the benchmark's CPU-baseline leg, never by the product path.
It shares no code with the GPU library.  Arguments are host arrays (torch CPU
tensors or numpy arrays); bf16 tensors are handed over as their raw 16-bit
patterns, fp8 E4M3 tensors as their raw 8-bit codes, and the C side widens
them exactly to fp64.

Method source: SkyRL blog "Scaling Training to 1M Token Context on
GLM-5.3-Flash", sections "DeepSeek Sparse Attention (DSA) Optimizations",
"Making Sparse Attention Actually Sparse" and "Splitting the DSA Indexer";
the readings the C file lists in its header apply here too.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_i64 = ctypes.c_int64
_int = ctypes.c_int
_ptr = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP over query rows, strict IEEE)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.dsa_oracle_bf16_value.restype = ctypes.c_double
        lib.dsa_oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.dsa_oracle_e4m3_value.restype = ctypes.c_double
        lib.dsa_oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.dsa_oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.dsa_oracle_e4m3_encode.argtypes = [ctypes.c_double]
        lib.dsa_oracle_pool_keys.restype = _int
        lib.dsa_oracle_pool_keys.argtypes = [_ptr, _ptr, _i64, _int, _int, _ptr]
        lib.dsa_oracle_pool_keys_fp8.restype = _int
        lib.dsa_oracle_pool_keys_fp8.argtypes = [_ptr, _ptr, _i64, _int, _int, _ptr, _ptr]
        lib.dsa_oracle_index_scores.restype = _int
        lib.dsa_oracle_index_scores.argtypes = [
            _ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _int, _int, _int, _ptr, _i64, _ptr]
        lib.dsa_oracle_index_topk.restype = _int
        lib.dsa_oracle_index_topk.argtypes = [
            _ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _int, _int, _int, _int, _ptr, _i64,
            _ptr, _ptr]
        lib.dsa_oracle_index_scores_fp8.restype = _int
        lib.dsa_oracle_index_scores_fp8.argtypes = [
            _ptr, _ptr, _ptr, ctypes.c_float, ctypes.c_float, _ptr, _i64, _i64, _i64, _i64, _int,
            _int, _int, _ptr, _i64, _ptr]
        lib.dsa_oracle_index_topk_fp8.restype = _int
        lib.dsa_oracle_index_topk_fp8.argtypes = [
            _ptr, _ptr, _ptr, ctypes.c_float, ctypes.c_float, _ptr, _i64, _i64, _i64, _i64, _int,
            _int, _int, _int, _ptr, _i64, _ptr, _ptr]
        lib.dsa_oracle_sparse_attn.restype = _int
        lib.dsa_oracle_sparse_attn.argtypes = [
            _ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _int, _int, _int, _int, _int, _int,
            ctypes.c_double, _ptr, _i64, _ptr, _ptr]
        lib.dsa_oracle_sparse_attn_bwd.restype = _int
        lib.dsa_oracle_sparse_attn_bwd.argtypes = [
            _ptr, _ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _int, _int, _int, _int, _int, _int,
            ctypes.c_double, _ptr, _i64, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr]
        lib.dsa_oracle_token_count.restype = _i64
        lib.dsa_oracle_token_count.argtypes = [_ptr, _i64, _i64, _int, _int, _int, _ptr, _i64]
        _lib = lib
        return lib


# ---------------------------------------------------------------- helpers

def _bits16(x) -> np.ndarray:
    """Raw 16-bit patterns of a bf16 tensor (torch) or a uint16 array."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    import torch
    assert x.dtype == torch.bfloat16, x.dtype
    return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def _codes8(x) -> np.ndarray:
    """Raw 8-bit codes of an fp8 E4M3 tensor (torch) or a uint8 array."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint8
        return np.ascontiguousarray(x)
    import torch
    assert x.dtype == torch.float8_e4m3fn, x.dtype
    return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.uint8).numpy())


def _f32(x) -> np.ndarray:
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x, dtype=np.float32)
    return np.ascontiguousarray(x.detach().cpu().float().numpy())


def _rows(rows, s_q) -> np.ndarray:
    if rows is None:
        return np.arange(s_q, dtype=np.int64)
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _w_args(w, h_idx):
    """w is [h_idx] (one row for every query, stride 0) or [s_q, h_idx]."""
    w32 = _f32(w)
    if w32.ndim == 1:
        assert w32.shape[0] == h_idx
        return w32, 0
    assert w32.shape[1] == h_idx
    return w32, h_idx


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


# ---------------------------------------------------------------- formats

def bf16_value(bits: int) -> float:
    return _load().dsa_oracle_bf16_value(bits)


def e4m3_value(code: int) -> float:
    return _load().dsa_oracle_e4m3_value(code)


def e4m3_encode(x: float) -> int:
    return _load().dsa_oracle_e4m3_encode(float(x))


# ---------------------------------------------------------------- indexer

def _gate(gate, s_k):
    """Per-token gates as contiguous fp32 [s_k], or None (mean pooling)."""
    if gate is None:
        return None
    g = np.ascontiguousarray(_f32(gate)).reshape(-1)
    if g.shape[0] != s_k:
        raise ValueError(f"gate has {g.shape[0]} entries for {s_k} keys")
    return g


def _pg(g):
    return None if g is None else _p(g)


def pool_keys(k_idx, pool: int = 4, gate=None) -> np.ndarray:
    """fp64 pooled keys [floor(S_k/pool), D_I] from bf16 keys [S_k, D_I]: the
    mean of each pool's rows, or with per-token gates [S_k] their gate-weighted
    sum."""
    kb = _bits16(k_idx)
    s_k, d = kb.shape
    g = _gate(gate, s_k)
    out = np.zeros((s_k // pool, d), dtype=np.float64)
    _check(_load().dsa_oracle_pool_keys(_p(kb), _pg(g), s_k, d, pool, _p(out)), "pool_keys")
    return out


def pool_keys_fp8(k8, pool: int = 4, gate=None):
    """Re-quantised fp8 pooled keys: (codes [P, D_I] uint8, exponents [P] int32)."""
    kc = _codes8(k8)
    s_k, d = kc.shape
    g = _gate(gate, s_k)
    codes = np.zeros((s_k // pool, d), dtype=np.uint8)
    exps = np.zeros((s_k // pool,), dtype=np.int32)
    _check(_load().dsa_oracle_pool_keys_fp8(_p(kc), _pg(g), s_k, d, pool, _p(codes), _p(exps)),
           "pool_keys_fp8")
    return codes, exps


def index_scores(q_idx, k_idx, w, q_pos0: int = 0, rows=None, pool: int = 4,
                 gate=None) -> np.ndarray:
    """fp32 scores [len(rows), P] (-inf where a pool is not eligible).

    q_idx [S_q, H_I, D_I] bf16, k_idx [S_k, D_I] bf16, w [H_I] or [S_q, H_I]."""
    qb, kb = _bits16(q_idx), _bits16(k_idx)
    s_q, h_idx, d_idx = qb.shape
    s_k = kb.shape[0]
    w32, ws = _w_args(w, h_idx)
    r = _rows(rows, s_q)
    g = _gate(gate, s_k)
    out = np.zeros((len(r), s_k // pool), dtype=np.float32)
    _check(_load().dsa_oracle_index_scores(
        _p(qb), _p(kb), _pg(g), _p(w32), ws, s_q, s_k, q_pos0, h_idx, d_idx, pool, _p(r), len(r),
        _p(out)), "index_scores")
    return out


def index_topk(q_idx, k_idx, w, k_pools: int, q_pos0: int = 0, rows=None, pool: int = 4,
               gate=None):
    """(idx int32 [len(rows), k_pools], selected fp32 scores [len(rows), k_pools])."""
    qb, kb = _bits16(q_idx), _bits16(k_idx)
    s_q, h_idx, d_idx = qb.shape
    s_k = kb.shape[0]
    w32, ws = _w_args(w, h_idx)
    r = _rows(rows, s_q)
    g = _gate(gate, s_k)
    idx = np.zeros((len(r), k_pools), dtype=np.int32)
    sc = np.zeros((len(r), k_pools), dtype=np.float32)
    _check(_load().dsa_oracle_index_topk(
        _p(qb), _p(kb), _pg(g), _p(w32), ws, s_q, s_k, q_pos0, h_idx, d_idx, pool, k_pools, _p(r),
        len(r), _p(idx), _p(sc)), "index_topk")
    return idx, sc


def index_scores_fp8(q8, k8, w, q_scale: float = 1.0, k_scale: float = 1.0, q_pos0: int = 0,
                     rows=None, pool: int = 4, gate=None) -> np.ndarray:
    qc, kc = _codes8(q8), _codes8(k8)
    s_q, h_idx, d_idx = qc.shape
    s_k = kc.shape[0]
    w32, ws = _w_args(w, h_idx)
    r = _rows(rows, s_q)
    g = _gate(gate, s_k)
    out = np.zeros((len(r), s_k // pool), dtype=np.float32)
    _check(_load().dsa_oracle_index_scores_fp8(
        _p(qc), _p(kc), _pg(g), q_scale, k_scale, _p(w32), ws, s_q, s_k, q_pos0, h_idx, d_idx, pool,
        _p(r), len(r), _p(out)), "index_scores_fp8")
    return out


def index_topk_fp8(q8, k8, w, k_pools: int, q_scale: float = 1.0, k_scale: float = 1.0,
                   q_pos0: int = 0, rows=None, pool: int = 4, gate=None):
    qc, kc = _codes8(q8), _codes8(k8)
    s_q, h_idx, d_idx = qc.shape
    s_k = kc.shape[0]
    w32, ws = _w_args(w, h_idx)
    r = _rows(rows, s_q)
    g = _gate(gate, s_k)
    idx = np.zeros((len(r), k_pools), dtype=np.int32)
    sc = np.zeros((len(r), k_pools), dtype=np.float32)
    _check(_load().dsa_oracle_index_topk_fp8(
        _p(qc), _p(kc), _pg(g), q_scale, k_scale, _p(w32), ws, s_q, s_k, q_pos0, h_idx, d_idx, pool,
        k_pools, _p(r), len(r), _p(idx), _p(sc)), "index_topk_fp8")
    return idx, sc


# ---------------------------------------------------------------- attention

def sparse_attn(q, k, v, idx_rows, k_pools: int, q_pos0: int = 0, rows=None, n_tail: int = 0,
                scale: float | None = None, pool: int = 4):
    """(o fp64 [len(rows), H, Dv], lse fp64 [len(rows), H]).

    q [S_q, H, D] bf16; k [S_k, D], v [S_k, Dv] bf16; idx_rows int32
    [len(rows), k_pools] holds the pool ids for the listed rows."""
    qb, kb, vb = _bits16(q), _bits16(k), _bits16(v)
    s_q, h, d = qb.shape
    s_k, dv = vb.shape
    assert kb.shape == (s_k, d)
    r = _rows(rows, s_q)
    ix = np.ascontiguousarray(np.asarray(idx_rows, dtype=np.int32))
    assert ix.shape == (len(r), k_pools), (ix.shape, len(r), k_pools)
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    o = np.zeros((len(r), h, dv), dtype=np.float64)
    lse = np.zeros((len(r), h), dtype=np.float64)
    _check(_load().dsa_oracle_sparse_attn(
        _p(qb), _p(kb), _p(vb), _p(ix), s_q, s_k, q_pos0, h, d, dv, k_pools, pool, n_tail,
        float(scale), _p(r), len(r), _p(o), _p(lse)), "sparse_attn")
    return o, lse


def sparse_attn_bwd(q, k, v, idx_rows, dout, k_pools: int, q_pos0: int = 0, rows=None,
                    n_tail: int = 0, scale: float | None = None, pool: int = 4,
                    magnitudes: bool = False):
    """Gradients of ``sparse_attn`` for the loss sum(dout . o) over the listed
    rows (dout of every other row taken as zero).

    q [S_q, H, D], k [S_k, D], v [S_k, Dv], dout [S_q, H, Dv] bf16; idx_rows
    int32 [len(rows), k_pools].  Returns dict with fp64 arrays dq
    [len(rows), H, D], dk [S_k, D], dv [S_k, Dv] and, with magnitudes=True,
    dq_mag, dk_mag, dv_mag of the same shapes (sums of absolute values the C
    file defines)."""
    qb, kb, vb, gb = _bits16(q), _bits16(k), _bits16(v), _bits16(dout)
    s_q, h, d = qb.shape
    s_k, dv = vb.shape
    assert kb.shape == (s_k, d) and gb.shape == (s_q, h, dv)
    r = _rows(rows, s_q)
    ix = np.ascontiguousarray(np.asarray(idx_rows, dtype=np.int32))
    assert ix.shape == (len(r), k_pools), (ix.shape, len(r), k_pools)
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    out = {"dq": np.zeros((len(r), h, d)), "dk": np.zeros((s_k, d)), "dv": np.zeros((s_k, dv))}
    if magnitudes:
        out.update(dq_mag=np.zeros((len(r), h, d)), dk_mag=np.zeros((s_k, d)),
                   dv_mag=np.zeros((s_k, dv)))
    m = (lambda n: _p(out[n]) if magnitudes else None)
    _check(_load().dsa_oracle_sparse_attn_bwd(
        _p(qb), _p(kb), _p(vb), _p(ix), _p(gb), s_q, s_k, q_pos0, h, d, dv, k_pools, pool,
        n_tail, float(scale), _p(r), len(r), _p(out["dq"]), _p(out["dk"]), _p(out["dv"]),
        m("dq_mag"), m("dk_mag"), m("dv_mag")), "sparse_attn_bwd")
    return out


def token_count(idx_rows, q_pos0: int, s_k: int, k_pools: int, rows, n_tail: int = 0,
                pool: int = 4) -> int:
    r = _rows(rows, None)
    ix = np.ascontiguousarray(np.asarray(idx_rows, dtype=np.int32))
    return int(_load().dsa_oracle_token_count(_p(ix), q_pos0, s_k, k_pools, pool, n_tail,
                                              _p(r), len(r)))
