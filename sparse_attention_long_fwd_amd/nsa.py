"""Thin ctypes binding of libnsa.so: same entry-point names as include/nsa.h.

Argument marshalling only.  Every step of the layer runs in the HIP kernels of
libnsa.so; PyTorch supplies device memory and the current stream.  The library
must be built (``python -m sparse_attention_long_fwd_amd.build``): loading
raises if it is missing, and there is no other execution path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# NSA_LIB_PATH selects another build of the same library (the host-sanitizer test's instrumented
# build); by default the in-tree libnsa.so.
LIB_PATH = os.environ.get("NSA_LIB_PATH") or os.path.join(_PKG, "libnsa.so")

NSA_OK, NSA_ERR_INVALID_ARG, NSA_ERR_UNSUPPORTED, NSA_ERR_HIP, NSA_ERR_WORKSPACE_TOO_SMALL = 0, -1, -2, -3, -4
NSA_F32, NSA_BF16 = 0, 1


class NsaShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("q_len", ctypes.c_int64), ("kv_len", ctypes.c_int64),
                ("q_start", ctypes.c_int64), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32)]


class NsaParams(ctypes.Structure):
    _fields_ = [("cmp_block", ctypes.c_int32), ("cmp_stride", ctypes.c_int32), ("sel_block", ctypes.c_int32),
                ("top_n", ctypes.c_int32), ("n_init", ctypes.c_int32), ("n_local", ctypes.c_int32),
                ("window", ctypes.c_int32), ("scale", ctypes.c_float)]


class NsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (status_string(status) if _lib else status, msg))
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I32, _I64, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SH, _PR = ctypes.POINTER(NsaShape), ctypes.POINTER(NsaParams)

EXPORTS = {
    "nsa_status_string": (ctypes.c_char_p, [_I32]),
    "nsa_last_error": (ctypes.c_char_p, []),
    "nsa_num_cmp_blocks": (_I64, [_I64, _I32, _I32]),
    "nsa_num_sel_blocks": (_I64, [_I64, _I32]),
    "nsa_compress_kv": (_I32, [_P, _P, _I32, _I64, _I64, _I32, _I32, _P, _P, _I32, _I32, _P, _P, _P]),
    "nsa_cmp_attn_scores": (_I32, [_P, _P, _P, _I32, _SH, _PR, _P, _P, _P, _P, _P]),
    "nsa_topk_blocks": (_I32, [_P, _SH, _PR, _P, _P, _P]),
    "nsa_sparse_attn_workspace_size": (_SZ, [_SH, _PR, _I32]),
    "nsa_sparse_attn_fwd": (_I32, [_P, _P, _P, _I32, _SH, _PR, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "nsa_hybrid_layer_workspace_size": (_SZ, [_SH, _PR, _I32]),
    "nsa_hybrid_layer_workspace_size_rows": (_SZ, [_SH, _PR, _I32, _I64]),
    "nsa_hybrid_layer_fwd": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _SH, _PR, _P, _P, _P, _P, _P, _P,
                                    _SZ, _P]),
    "nsa_decode_workspace_size": (_SZ, [_SH, _PR, _I32]),
    "nsa_decode_fwd": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _SH, _PR, _P, _P, _I32, _I64, _P, _P, _P, _P, _P,
                              _P, _SZ, _P]),
    "nsa_decode_fwd_noalloc": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _SH, _PR, _P, _P, _I32, _I64, _P, _P, _P, _P,
                                      _P, _P]),
    "nsa_compress_append": (_I32, [_P, _P, _I32, _I64, _I64, _I32, _I32, _P, _P, _I32, _I32, _P, _P, _I32, _I64,
                                   _I32, _P, _P, _P]),
    "nsa_gate_proj": (_I32, [_P, _P, _P, _I32, _I64, _I64, _I32, _I32, _P, _P]),
    "nsa_hybrid_layer_fwd_branch_kv": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _SH, _PR,
                                              _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "nsa_hybrid_layer_bwd_workspace_size": (_SZ, [_SH, _PR, _I32]),
    "nsa_hybrid_layer_bwd": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _SH, _PR, _P, _P, _P, _P, _P, _P, _P,
                                    _SZ, _P]),
    "nsa_set_force_generic": (_I32, [_I32]),
    "nsa_profile_enable": (_I32, [_I32]),
    "nsa_profile_read": (_I32, [ctypes.POINTER(ctypes.c_float), _I32]),
}


def lib():
    """Load libnsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libnsa.so is not built: run `python -m sparse_attention_long_fwd_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().nsa_status_string(status).decode()


def last_error() -> str:
    return lib().nsa_last_error().decode()


def _check(status: int):
    if status != NSA_OK:
        raise NsaError(status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous(), "tensors must be contiguous device tensors"
    return t.data_ptr()


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return NSA_F32
    if t.dtype == torch.bfloat16:
        return NSA_BF16
    raise TypeError("q/k/v must be float32 or bfloat16, got %s" % t.dtype)


def make_shape(batch, q_len, kv_len, q_start, num_q_heads, num_kv_heads, head_dim) -> NsaShape:
    return NsaShape(batch, q_len, kv_len, q_start, num_q_heads, num_kv_heads, head_dim)


def make_params(cmp_block=32, cmp_stride=16, sel_block=64, top_n=16, n_init=1, n_local=2, window=512,
                scale=0.0) -> NsaParams:
    return NsaParams(cmp_block, cmp_stride, sel_block, top_n, n_init, n_local, window, scale)


def shape_of(q: torch.Tensor, k: torch.Tensor, q_start: int = 0) -> NsaShape:
    B, Tq, Hq, D = q.shape
    return make_shape(B, Tq, k.shape[1], q_start, Hq, k.shape[2], D)


def num_cmp_blocks(kv_len: int, cmp_block: int, cmp_stride: int) -> int:
    return int(lib().nsa_num_cmp_blocks(kv_len, cmp_block, cmp_stride))


def num_sel_blocks(kv_len: int, sel_block: int) -> int:
    return int(lib().nsa_num_sel_blocks(kv_len, sel_block))


def set_force_generic(on: bool) -> bool:
    return bool(lib().nsa_set_force_generic(1 if on else 0))


PHASES = ("compress", "cmp_attn_importance", "topk", "window_text", "selection_combine")


def profile_enable(on: bool = True):
    _check(lib().nsa_profile_enable(1 if on else 0))


def profile_read():
    """Phase durations (ms) of the last nsa_hybrid_layer_fwd, after profile_enable()."""
    buf = (ctypes.c_float * 8)()
    n = lib().nsa_profile_read(buf, 8)
    if n < 0:
        _check(n)
    return list(buf[:n])


def nsa_compress_kv(k, v, w_k, w_v, cmp_block=32, cmp_stride=16, k_cmp=None, v_cmp=None, stream=None):
    B, T, H, D = k.shape
    Nc = num_cmp_blocks(T, cmp_block, cmp_stride)
    if k_cmp is None:
        k_cmp = torch.empty(B, Nc, H, D, dtype=k.dtype, device=k.device)
    if v_cmp is None:
        v_cmp = torch.empty(B, Nc, H, D, dtype=v.dtype, device=v.device)
    _check(lib().nsa_compress_kv(_ptr(k), _ptr(v), _dtype_code(k), B, T, H, D, _ptr(w_k), _ptr(w_v), cmp_block,
                                 cmp_stride, _ptr(k_cmp), _ptr(v_cmp), _stream(stream)))
    return k_cmp, v_cmp


def nsa_cmp_attn_scores(q, k_cmp, v_cmp, shape: NsaShape, params: NsaParams, is_video=None, o_cmp=None,
                        lse=None, importance=None, want=("o_cmp", "lse", "importance"), stream=None):
    B, Tq, Hq, D = q.shape
    Ns = num_sel_blocks(shape.kv_len, params.sel_block)
    if o_cmp is None and "o_cmp" in want:
        o_cmp = torch.zeros_like(q)
    if lse is None and "lse" in want:
        lse = torch.zeros(B, Tq, Hq, dtype=torch.float32, device=q.device)
    if importance is None and "importance" in want:
        importance = torch.zeros(B, Tq, shape.num_kv_heads, Ns, dtype=torch.float32, device=q.device)
    _check(lib().nsa_cmp_attn_scores(_ptr(q), _ptr(k_cmp), _ptr(v_cmp), _dtype_code(q), ctypes.byref(shape),
                                     ctypes.byref(params), _ptr(is_video), _ptr(o_cmp), _ptr(lse),
                                     _ptr(importance), _stream(stream)))
    return o_cmp, lse, importance


def nsa_topk_blocks(importance, shape: NsaShape, params: NsaParams, is_video=None, block_idx=None, stream=None):
    B, Tq, Hkv, _ = importance.shape
    if block_idx is None:
        block_idx = torch.full((B, Tq, Hkv, params.top_n), -1, dtype=torch.int32, device=importance.device)
    _check(lib().nsa_topk_blocks(_ptr(importance), ctypes.byref(shape), ctypes.byref(params), _ptr(is_video),
                                 _ptr(block_idx), _stream(stream)))
    return block_idx


def nsa_sparse_attn_workspace_size(shape: NsaShape, params: NsaParams, dtype_code: int) -> int:
    return int(lib().nsa_sparse_attn_workspace_size(ctypes.byref(shape), ctypes.byref(params), dtype_code))


def nsa_sparse_attn_fwd(q, k, v, shape: NsaShape, params: NsaParams, block_idx, is_video=None, o_cmp=None,
                        gates=None, out=None, o_slc=None, o_swa=None, workspace=None, stream=None):
    dt = _dtype_code(q)
    ws_bytes = nsa_sparse_attn_workspace_size(shape, params, dt)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    _check(lib().nsa_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), dt, ctypes.byref(shape), ctypes.byref(params),
                                     _ptr(block_idx), _ptr(is_video), _ptr(o_cmp), _ptr(gates), _ptr(out),
                                     _ptr(o_slc), _ptr(o_swa), _ptr(workspace),
                                     0 if workspace is None else workspace.numel(), _stream(stream)))
    return out, o_slc, o_swa


def nsa_hybrid_layer_workspace_size(shape: NsaShape, params: NsaParams, dtype_code: int) -> int:
    return int(lib().nsa_hybrid_layer_workspace_size(ctypes.byref(shape), ctypes.byref(params), dtype_code))


def nsa_hybrid_layer_workspace_size_rows(shape: NsaShape, params: NsaParams, dtype_code: int,
                                         rows_per_chunk: int) -> int:
    return int(lib().nsa_hybrid_layer_workspace_size_rows(ctypes.byref(shape), ctypes.byref(params), dtype_code,
                                                          rows_per_chunk))


def _layer_workspace(shape, params, dt, rows_per_chunk, device):
    n = (nsa_hybrid_layer_workspace_size(shape, params, dt) if rows_per_chunk is None else
         nsa_hybrid_layer_workspace_size_rows(shape, params, dt, rows_per_chunk))
    return torch.empty(n, dtype=torch.uint8, device=device)


def nsa_hybrid_layer_fwd(q, k, v, gates, shape: NsaShape, params: NsaParams, w_k=None, w_v=None, k_cmp_in=None,
                         v_cmp_in=None, is_video=None, out=None, o_cmp=None, o_slc=None, o_swa=None,
                         block_idx_out=None, workspace=None, stream=None, rows_per_chunk=None):
    """rows_per_chunk (when no workspace is given): size the workspace for passes of at most that many
    rows (0: one pass); None: the library's default size."""
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = _layer_workspace(shape, params, dt, rows_per_chunk, q.device)
    _check(lib().nsa_hybrid_layer_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(k_cmp_in), _ptr(v_cmp_in), _ptr(w_k),
                                      _ptr(w_v), _ptr(gates), _ptr(is_video), dt, ctypes.byref(shape),
                                      ctypes.byref(params), _ptr(out), _ptr(o_cmp), _ptr(o_slc), _ptr(o_swa),
                                      _ptr(block_idx_out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


PAGE_ROWS = 64  # tokens per page of a paged K / V cache


def nsa_decode_workspace_size(shape: NsaShape, params: NsaParams, dtype_code: int) -> int:
    return int(lib().nsa_decode_workspace_size(ctypes.byref(shape), ctypes.byref(params), dtype_code))


def nsa_decode_fwd(q, k, v, k_cmp, v_cmp, gates, shape: NsaShape, params: NsaParams, kv_lens=None,
                   page_table=None, num_pages=0, is_video=None, out=None, o_cmp=None, o_slc=None, o_swa=None,
                   block_idx_out=None, workspace=None, stream=None):
    """One decode row per sequence; kv_lens [B] int32, page_table [B, max_pages] int32 (k, v then a page pool)."""
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = torch.empty(nsa_decode_workspace_size(shape, params, dt), dtype=torch.uint8, device=q.device)
    max_pages = 0 if page_table is None else page_table.shape[1]
    if page_table is not None and not num_pages:
        num_pages = k.shape[0]
    _check(lib().nsa_decode_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(k_cmp), _ptr(v_cmp), _ptr(gates), _ptr(is_video),
                                dt, ctypes.byref(shape), ctypes.byref(params), _ptr(kv_lens), _ptr(page_table),
                                max_pages, num_pages, _ptr(out), _ptr(o_cmp), _ptr(o_slc), _ptr(o_swa),
                                _ptr(block_idx_out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def nsa_decode_fwd_noalloc(q, k, v, k_cmp, v_cmp, gates, shape: NsaShape, params: NsaParams, kv_lens=None,
                           page_table=None, num_pages=0, is_video=None, out=None, o_cmp=None, o_slc=None,
                           o_swa=None, block_idx_out=None, stream=None):
    """nsa_decode_fwd with the library's own device scratch instead of a workspace (the call allocates
    nothing on the device; `out` must then be given by the caller to keep it that way)."""
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    max_pages = 0 if page_table is None else page_table.shape[1]
    if page_table is not None and not num_pages:
        num_pages = k.shape[0]
    _check(lib().nsa_decode_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(k_cmp), _ptr(v_cmp), _ptr(gates),
                                        _ptr(is_video), dt, ctypes.byref(shape), ctypes.byref(params), _ptr(kv_lens),
                                        _ptr(page_table), max_pages, num_pages, _ptr(out), _ptr(o_cmp), _ptr(o_slc),
                                        _ptr(o_swa), _ptr(block_idx_out), _stream(stream)))
    return out


def nsa_compress_append(k, v, w_k, w_v, k_cmp, v_cmp, kv_len, n_new, kv_lens=None, page_table=None, num_pages=0,
                        cmp_block=32, cmp_stride=16, stream=None):
    """Writes the compressed blocks completed by the last n_new tokens of every sequence."""
    B, _, H, D = k_cmp.shape
    max_pages = 0 if page_table is None else page_table.shape[1]
    if page_table is not None and not num_pages:
        num_pages = k.shape[0]
    _check(lib().nsa_compress_append(_ptr(k), _ptr(v), _dtype_code(k), B, kv_len, H, D, _ptr(w_k), _ptr(w_v),
                                     cmp_block, cmp_stride, _ptr(kv_lens), _ptr(page_table), max_pages, num_pages,
                                     n_new, _ptr(k_cmp), _ptr(v_cmp), _stream(stream)))
    return k_cmp, v_cmp


def nsa_gate_proj(x, w_g, b_g=None, gates=None, stream=None):
    """Branch gates [B, T, Hq, 3] (fp32) from hidden states x [B, T, hidden] and w_g [3 Hq, hidden]."""
    B, T, K = x.shape
    Hq = w_g.shape[0] // 3
    if gates is None:
        gates = torch.empty(B, T, Hq, 3, dtype=torch.float32, device=x.device)
    _check(lib().nsa_gate_proj(_ptr(x), _ptr(w_g), _ptr(b_g), _dtype_code(x), B, T, K, Hq, _ptr(gates),
                               _stream(stream)))
    return gates


def nsa_hybrid_layer_fwd_branch_kv(q, kv_c, kv_s, kv_w, gates, shape: NsaShape, params: NsaParams, w_k=None,
                                   w_v=None, k_cmp_in=None, v_cmp_in=None, is_video=None, out=None, o_cmp=None,
                                   o_slc=None, o_swa=None, block_idx_out=None, workspace=None, stream=None,
                                   rows_per_chunk=None):
    """The layer with keys / values per branch: kv_c (compression), kv_s (selection), kv_w (window and
    text rows), each a (k, v) pair; rows_per_chunk as for nsa_hybrid_layer_fwd."""
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = _layer_workspace(shape, params, dt, rows_per_chunk, q.device)
    _check(lib().nsa_hybrid_layer_fwd_branch_kv(
        _ptr(q), _ptr(kv_c[0]), _ptr(kv_c[1]), _ptr(kv_s[0]), _ptr(kv_s[1]), _ptr(kv_w[0]), _ptr(kv_w[1]),
        _ptr(k_cmp_in), _ptr(v_cmp_in), _ptr(w_k), _ptr(w_v), _ptr(gates), _ptr(is_video), dt, ctypes.byref(shape),
        ctypes.byref(params), _ptr(out), _ptr(o_cmp), _ptr(o_slc), _ptr(o_swa), _ptr(block_idx_out),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def nsa_hybrid_layer_bwd_workspace_size(shape: NsaShape, params: NsaParams, dtype_code: int) -> int:
    return int(lib().nsa_hybrid_layer_bwd_workspace_size(ctypes.byref(shape), ctypes.byref(params), dtype_code))


def nsa_hybrid_layer_bwd(q, k, v, gates, block_idx, d_out, shape: NsaShape, params: NsaParams, w_k=None, w_v=None,
                         is_video=None, workspace=None, stream=None):
    """Gradients of sum(d_out * out): returns dict dq, dk, dv, d_gates, dw_k, dw_v (fp32)."""
    dt = _dtype_code(q)
    dev = q.device
    f32 = torch.float32
    g = dict(dq=torch.empty(q.shape, dtype=f32, device=dev), dk=torch.empty(k.shape, dtype=f32, device=dev),
             dv=torch.empty(v.shape, dtype=f32, device=dev), d_gates=torch.empty(gates.shape, dtype=f32, device=dev),
             dw_k=torch.empty(params.cmp_block, dtype=f32, device=dev),
             dw_v=torch.empty(params.cmp_block, dtype=f32, device=dev))
    if workspace is None:
        workspace = torch.empty(max(1, nsa_hybrid_layer_bwd_workspace_size(shape, params, dt)), dtype=torch.uint8,
                                device=dev)
    _check(lib().nsa_hybrid_layer_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(w_k), _ptr(w_v), _ptr(gates), _ptr(is_video),
                                      _ptr(block_idx), _ptr(d_out), dt, ctypes.byref(shape), ctypes.byref(params),
                                      _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["d_gates"]),
                                      _ptr(g["dw_k"]), _ptr(g["dw_v"]), _ptr(workspace), workspace.numel(),
                                      _stream(stream)))
    return g
