"""fp64 CPU oracle of the VideoNSA hybrid attention layer (forward).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The product library never imports it.

The arithmetic lives in ``nsa_oracle.c`` (plain C, fp64, OpenMP over rows).
This module builds it with gcc, loads it with ctypes and composes the layer
with numpy, step by step:

1. compress K and V into block tokens (top168.com digest, section 一: the
   compression branch);
2. for video rows, compression-branch attention and block importance;
3. top-n block choice per (row, KV group) with forced blocks;
4. selection-branch and sliding-window attention;
5. gated sum of the three branch outputs (csdn page, section 3.1: three gate
   values per head weight the branches; here the given sigmoid values are used
   as they are, without normalisation);
6. text rows: dense causal attention, ungated (shd-paper.top page, English
   abstract: dense attention for text, NSA for video).

Every function takes and returns numpy arrays.  Inputs are float32 arrays that
hold the exact input values (bf16 values widen exactly); outputs are float64.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libnsa_oracle.so")
# NSA_ORACLE_LIB_PATH loads another, prebuilt copy of this oracle (the host-sanitizer test's
# instrumented build) instead of building and loading the default one.
_LIB_OVERRIDE = os.environ.get("NSA_ORACLE_LIB_PATH")
_lib = None

_i64 = ctypes.c_int64
_dbl = ctypes.c_double
_p = ctypes.c_void_p


def build(force: bool = False) -> str:
    """Compile the oracle shared library with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            L = ctypes.CDLL(_LIB_PATH)
        L.oracle_num_cmp_blocks.restype = _i64
        L.oracle_num_cmp_blocks.argtypes = [_i64, _i64, _i64]
        L.oracle_num_sel_blocks.restype = _i64
        L.oracle_num_sel_blocks.argtypes = [_i64, _i64]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_compress.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _i64, _p]
        L.oracle_cmp_rows.argtypes = [_p, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                      _i64, _dbl, _p, _p, _p]
        L.oracle_topk_rows.argtypes = [_p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _p, _p]
        L.oracle_sparse_rows.argtypes = [_p, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _i64, _p, _i64,
                                         _i64, _dbl, _p, _p]
        L.oracle_dense_rows.argtypes = [_p, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _dbl, _p, _p]
        L.oracle_gate_proj.argtypes = [_p, _i64, _i64, _p, _i64, _p, _p]
        L.oracle_layer_bwd.argtypes = [_p, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _i64, _p, _p, _i64,
                                       _i64, _i64, _p, _i64, _i64, _dbl, _p, _p, _p, _p, _p, _p, _p, _p, _p]
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def num_cmp_blocks(T: int, l: int, d: int) -> int:
    return int(lib().oracle_num_cmp_blocks(T, l, d))


def num_sel_blocks(T: int, ls: int) -> int:
    return int(lib().oracle_num_sel_blocks(T, ls))


def default_scale(D: int, scale: float = 0.0) -> float:
    return scale if scale > 0 else 1.0 / math.sqrt(D)


def compress(x, w, l: int, d: int) -> np.ndarray:
    """x [T, H, D] -> [Nc, H, D] fp64 positional weighted sums."""
    x = _f32(x)
    w = _f32(w)
    T, H, D = x.shape
    out = np.zeros((num_cmp_blocks(T, l, d), H, D), dtype=np.float64)
    lib().oracle_compress(_ptr(x), T, H, D, _ptr(w), l, d, _ptr(out))
    return out


def cmp_rows(q_rows, pos, kc, vc, Hq: int, l: int, d: int, ls: int, T: int, scale: float):
    """Compression-branch output, log-sum-exp and block importance for the given rows."""
    q_rows = _f32(q_rows)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    kc = np.ascontiguousarray(kc, dtype=np.float64)
    vc = np.ascontiguousarray(vc, dtype=np.float64)
    R = pos.shape[0]
    Nc, Hkv, D = kc.shape
    Ns = num_sel_blocks(T, ls)
    o = np.zeros((R, Hq, D), dtype=np.float64)
    lse = np.zeros((R, Hq), dtype=np.float64)
    imp = np.zeros((R, Hkv, Ns), dtype=np.float64)
    lib().oracle_cmp_rows(_ptr(q_rows), _ptr(pos), R, _ptr(kc), _ptr(vc), Nc, Hq, Hkv, D, l, d, ls, Ns,
                          scale, _ptr(o), _ptr(lse), _ptr(imp))
    return o, lse, imp


def topk_rows(imp, pos, ls: int, n: int, n_init: int, n_local: int):
    """Chosen blocks [R, Hkv, n] (ascending, -1 padded) and the selection gap [R, Hkv]."""
    imp = np.ascontiguousarray(imp, dtype=np.float64)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    R, Hkv, Ns = imp.shape
    idx = np.full((R, Hkv, n), -1, dtype=np.int32)
    gap = np.zeros((R, Hkv), dtype=np.float64)
    lib().oracle_topk_rows(_ptr(imp), _ptr(pos), R, Hkv, Ns, ls, n, n_init, n_local, _ptr(idx), _ptr(gap))
    return idx, gap


def sparse_rows(q_rows, pos, k, v, idx, ls: int, w: int, scale: float, slc=True, swa=True):
    """Selection-branch and sliding-window outputs [R, Hq, D] for the given rows."""
    q_rows = _f32(q_rows)
    k = _f32(k)
    v = _f32(v)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    R, Hq, D = q_rows.shape
    T, Hkv, _ = k.shape
    n = idx.shape[2]
    o_slc = np.zeros((R, Hq, D), dtype=np.float64) if slc else None
    o_swa = np.zeros((R, Hq, D), dtype=np.float64) if swa else None
    lib().oracle_sparse_rows(_ptr(q_rows), _ptr(pos), R, _ptr(k), _ptr(v), T, Hq, Hkv, D, ls, _ptr(idx), n, w,
                             scale, _ptr(o_slc), _ptr(o_swa))
    return o_slc, o_swa


def dense_rows(q_rows, pos, k, v, scale: float):
    """Dense causal attention [R, Hq, D] and its log-sum-exp [R, Hq] for the given rows."""
    q_rows = _f32(q_rows)
    k = _f32(k)
    v = _f32(v)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    R, Hq, D = q_rows.shape
    T, Hkv, _ = k.shape
    o = np.zeros((R, Hq, D), dtype=np.float64)
    lse = np.zeros((R, Hq), dtype=np.float64)
    lib().oracle_dense_rows(_ptr(q_rows), _ptr(pos), R, _ptr(k), _ptr(v), T, Hq, Hkv, D, scale, _ptr(o), _ptr(lse))
    return o, lse


def gate_proj(x, w, b=None) -> np.ndarray:
    """Gate values g = 1 / (1 + exp(-(x w^T + b))) for x [R, K], w [N, K], b [N] -> [R, N] fp64
    (column f = 3 h + c: head h, branch c in cmp, slc, swa order)."""
    x = _f32(x)
    w = _f32(w)
    b = None if b is None else _f32(b)
    R, K = x.shape
    N = w.shape[0]
    g = np.zeros((R, N), dtype=np.float64)
    lib().oracle_gate_proj(_ptr(x), R, K, _ptr(w), N, _ptr(b), _ptr(g))
    return g


def layer(q, k, v, w_k, w_v, gates, is_video, params: Dict, q_start: int = 0,
          rows: Optional[np.ndarray] = None, kc=None, vc=None, kv_slc=None, kv_swa=None) -> Dict[str, np.ndarray]:
    """The hybrid layer for one batch element.

    q [Tq, Hq, D], k/v [T, Hkv, D], gates [Tq, Hq, 3], is_video [Tq]; row r of q
    sits at absolute position q_start + r.  ``rows`` picks a subset of q's rows
    (default: all).  ``kc``/``vc`` replace the compression of k/v when given (a
    precomputed compressed cache).  ``kv_slc`` / ``kv_swa`` give the selection
    branch, and the window branch with the text rows, keys and values of their
    own (Native Sparse Attention's per-branch projections); by default all
    branches share k/v.  Returns fp64 arrays over the chosen rows:
    o_cmp, lse_cmp, imp, idx, gap, o_slc, o_swa (video rows; zero for text rows)
    and out (gated sum for video rows, dense causal attention for text rows).
    """
    q = np.asarray(q)
    Tq, Hq, D = q.shape
    T = k.shape[0]
    l, d, ls = params["cmp_block"], params["cmp_stride"], params["sel_block"]
    n, n_init, n_local, w = params["top_n"], params["n_init"], params["n_local"], params["window"]
    scale = default_scale(D, params.get("scale", 0.0))
    rows = np.arange(Tq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    pos = rows + q_start
    q_rows = _f32(q[rows])
    vid = np.asarray(is_video)[rows].astype(bool)
    if kc is None:
        kc = compress(k, w_k, l, d)
    if vc is None:
        vc = compress(v, w_v, l, d)
    R = rows.shape[0]
    Hkv = k.shape[1]
    Ns = num_sel_blocks(T, ls)
    res = dict(o_cmp=np.zeros((R, Hq, D)), lse_cmp=np.full((R, Hq), -np.inf), imp=np.zeros((R, Hkv, Ns)),
               idx=np.full((R, Hkv, n), -1, dtype=np.int32), gap=np.full((R, Hkv), np.inf),
               o_slc=np.zeros((R, Hq, D)), o_swa=np.zeros((R, Hq, D)), out=np.zeros((R, Hq, D)))
    vr = np.nonzero(vid)[0]
    tr = np.nonzero(~vid)[0]
    if vr.size:
        o_cmp, lse, imp = cmp_rows(q_rows[vr], pos[vr], kc, vc, Hq, l, d, ls, T, scale)
        idx, gap = topk_rows(imp, pos[vr], ls, n, n_init, n_local)
        ks, vs = kv_slc if kv_slc is not None else (k, v)
        kw, vw = kv_swa if kv_swa is not None else (k, v)
        o_slc, _ = sparse_rows(q_rows[vr], pos[vr], ks, vs, idx, ls, w, scale, swa=False)
        _, o_swa = sparse_rows(q_rows[vr], pos[vr], kw, vw, idx, ls, w, scale, slc=False)
        g = np.asarray(gates, dtype=np.float64)[rows[vr]]
        res["o_cmp"][vr], res["lse_cmp"][vr], res["imp"][vr] = o_cmp, lse, imp
        res["idx"][vr], res["gap"][vr] = idx, gap
        res["o_slc"][vr], res["o_swa"][vr] = o_slc, o_swa
        res["out"][vr] = g[..., 0:1] * o_cmp + g[..., 1:2] * o_slc + g[..., 2:3] * o_swa
    if tr.size:
        kw, vw = kv_swa if kv_swa is not None else (k, v)
        res["out"][tr], _ = dense_rows(q_rows[tr], pos[tr], kw, vw, scale)
    res["kc"], res["vc"] = kc, vc
    return res


def layer_bwd(q, k, v, w_k, w_v, gates, is_video, params: Dict, dout, q_start: int = 0,
              idx: Optional[np.ndarray] = None, rows: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Gradients of sum(dout * out) for the hybrid layer of one batch element.

    q, dout [Tq, Hq, D], k/v [T, Hkv, D], gates [Tq, Hq, 3], is_video [Tq], w_k / w_v [l].  The
    chosen blocks are held fixed (no gradient through top-n): ``idx`` [Tq, Hkv, n] when given, else
    the forward's own choice.  ``rows`` restricts the loss to those rows of q (dq and dgates are
    then those rows' own; dk, dv, dw_k, dw_v hold only their contributions).  Returns fp64 dq, dk,
    dv, dgates, dw_k, dw_v and the idx used.
    """
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        if idx is None:
            idx = layer(q, k, v, w_k, w_v, gates, is_video, params, q_start=q_start, rows=rows)["idx"]
        else:
            idx = np.asarray(idx)[rows]
        q, gates, dout = np.asarray(q)[rows], np.asarray(gates)[rows], np.asarray(dout)[rows]
        is_video = np.asarray(is_video)[rows]
        pos = (rows + q_start).astype(np.int64)
    else:
        pos = None
    q = _f32(q)
    k = _f32(k)
    v = _f32(v)
    Tq, Hq, D = q.shape
    T, Hkv, _ = k.shape
    l, d, ls = params["cmp_block"], params["cmp_stride"], params["sel_block"]
    n, w = params["top_n"], params["window"]
    scale = default_scale(D, params.get("scale", 0.0))
    if idx is None:
        idx = layer(q, k, v, w_k, w_v, gates, is_video, params, q_start=q_start)["idx"]
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    kc = compress(k, w_k, l, d)
    vc = compress(v, w_v, l, d)
    Nc = kc.shape[0]
    if pos is None:
        pos = np.arange(q_start, q_start + Tq, dtype=np.int64)
    vid = np.ascontiguousarray(is_video, dtype=np.uint8)
    out = dict(dq=np.zeros((Tq, Hq, D)), dk=np.zeros((T, Hkv, D)), dv=np.zeros((T, Hkv, D)),
               dgates=np.zeros((Tq, Hq, 3)), dw_k=np.zeros(l), dw_v=np.zeros(l))
    wk, wv, gg, do = _f32(w_k), _f32(w_v), _f32(gates), _f32(dout)  # kept alive through the call
    lib().oracle_layer_bwd(_ptr(q), _ptr(pos), Tq, _ptr(k), _ptr(v), T, Hq, Hkv, D, _ptr(kc), _ptr(vc), Nc,
                           _ptr(wk), _ptr(wv), l, d, ls, _ptr(idx), n, w, scale, _ptr(gg), _ptr(vid), _ptr(do),
                           _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dgates"]),
                           _ptr(out["dw_k"]), _ptr(out["dw_v"]))
    out["idx"] = idx
    return out
