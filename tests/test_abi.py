"""Host-only checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before launching anything (no GPU needed:
every call here fails validation on the host)."""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_attention_long_fwd_amd import nsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nsa.h")
FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nsa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = nsa.lib()
    decl = declared_symbols()
    assert len(decl) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", nsa.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for s in decl:
        assert s in exported, s
        assert hasattr(L, s)
    assert set(nsa.EXPORTS) == set(decl)


def test_status_strings_and_block_counts():
    assert nsa.status_string(0) == "NSA_OK"
    assert nsa.status_string(-4) == "NSA_ERR_WORKSPACE_TOO_SMALL"
    assert nsa.status_string(99) == "NSA_UNKNOWN_STATUS"
    assert nsa.num_cmp_blocks(131072, 32, 16) == 8191
    assert nsa.num_cmp_blocks(31, 32, 16) == 0
    assert nsa.num_cmp_blocks(36352, 32, 16) == 2271
    assert nsa.num_sel_blocks(131072, 64) == 2048 and nsa.num_sel_blocks(36352, 64) == 568
    assert nsa.num_sel_blocks(65, 64) == 2
    assert nsa.num_cmp_blocks(-1, 32, 16) == -1


def _shape(**kw):
    d = dict(batch=1, q_len=1024, kv_len=1024, q_start=0, num_q_heads=4, num_kv_heads=1, head_dim=64)
    d.update(kw)
    return nsa.make_shape(**d)


def _params(**kw):
    d = dict(cmp_block=32, cmp_stride=16, sel_block=64, top_n=4, n_init=1, n_local=2, window=128, scale=0.0)
    d.update(kw)
    return nsa.make_params(**d)


def _layer(shape, params, ws_bytes=1 << 40, out=FAKE, q=FAKE, dtype=nsa.NSA_F32, kc=None, vc=None):
    L = nsa.lib()
    return L.nsa_hybrid_layer_fwd(q, FAKE, FAKE, kc, vc, FAKE, FAKE, FAKE, None, dtype, ctypes.byref(shape),
                                  ctypes.byref(params), out, None, None, None, None, FAKE, ws_bytes, None)


@pytest.mark.parametrize("shape_kw,params_kw,code", [
    (dict(num_q_heads=6, num_kv_heads=4), {}, nsa.NSA_ERR_INVALID_ARG),
    (dict(q_start=10), {}, nsa.NSA_ERR_INVALID_ARG),                      # q_start + q_len > kv_len
    (dict(head_dim=60), {}, nsa.NSA_ERR_UNSUPPORTED),
    (dict(head_dim=512), {}, nsa.NSA_ERR_UNSUPPORTED),
    (dict(batch=-1), {}, nsa.NSA_ERR_INVALID_ARG),
    ({}, dict(top_n=2), nsa.NSA_ERR_INVALID_ARG),                         # top_n < n_init + n_local
    ({}, dict(top_n=33), nsa.NSA_ERR_UNSUPPORTED),
    ({}, dict(window=0), nsa.NSA_ERR_INVALID_ARG),
    ({}, dict(cmp_stride=0), nsa.NSA_ERR_INVALID_ARG),
    ({}, dict(n_local=0), nsa.NSA_ERR_INVALID_ARG),
    ({}, dict(scale=-1.0), nsa.NSA_ERR_INVALID_ARG),
])
def test_layer_rejects_bad_shapes_and_params(shape_kw, params_kw, code):
    assert _layer(_shape(**shape_kw), _params(**params_kw)) == code
    assert nsa.last_error() != ""


def test_layer_rejects_null_and_small_workspace():
    sh, pr = _shape(), _params()
    assert _layer(sh, pr, out=None) == nsa.NSA_ERR_INVALID_ARG
    assert _layer(sh, pr, q=None) == nsa.NSA_ERR_INVALID_ARG
    assert _layer(sh, pr, kc=FAKE) == nsa.NSA_ERR_INVALID_ARG        # k_cmp_in without v_cmp_in
    need = nsa.nsa_hybrid_layer_workspace_size(sh, pr, nsa.NSA_F32)
    assert need > 0
    assert _layer(sh, pr, ws_bytes=need - 1) == nsa.NSA_ERR_WORKSPACE_TOO_SMALL
    assert "workspace" in nsa.last_error()
    assert _layer(sh, pr, q=FAKE + 4) == nsa.NSA_ERR_INVALID_ARG     # misaligned
    assert nsa.nsa_hybrid_layer_workspace_size(_shape(num_kv_heads=3), pr, nsa.NSA_F32) == 0


def test_other_entry_points_validate_first():
    L = nsa.lib()
    sh, pr = _shape(), _params()
    assert L.nsa_compress_kv(FAKE, FAKE, 7, 1, 1024, 1, 64, FAKE, FAKE, 32, 16, FAKE, FAKE, None) == -1
    assert L.nsa_compress_kv(None, FAKE, 0, 1, 1024, 1, 64, FAKE, FAKE, 32, 16, FAKE, FAKE, None) == -1
    assert L.nsa_compress_kv(FAKE, FAKE, 0, 1, 1024, 1, 60, FAKE, FAKE, 32, 16, FAKE, FAKE, None) == -2
    # nothing to do: fewer tokens than one block
    assert L.nsa_compress_kv(None, None, 0, 1, 31, 1, 64, None, None, 32, 16, None, None, None) == 0
    assert L.nsa_cmp_attn_scores(FAKE, FAKE, FAKE, 0, ctypes.byref(sh), ctypes.byref(pr), None, None, None,
                                 None, None) == -1
    assert L.nsa_topk_blocks(FAKE, ctypes.byref(sh), ctypes.byref(_params(top_n=1)), None, FAKE, None) == -1
    assert L.nsa_topk_blocks(None, ctypes.byref(sh), ctypes.byref(pr), None, FAKE, None) == -1
    assert L.nsa_sparse_attn_fwd(FAKE, FAKE, FAKE, 0, ctypes.byref(sh), ctypes.byref(pr), FAKE, None, None, None,
                                 None, None, None, None, 0, None) == -1       # no output
    assert L.nsa_sparse_attn_fwd(FAKE, FAKE, FAKE, 0, ctypes.byref(sh), ctypes.byref(pr), FAKE, None, None, FAKE,
                                 FAKE, None, None, None, 0, None) == -1       # out without o_cmp
    # empty problems launch nothing and succeed
    e = _shape(q_len=0)
    assert L.nsa_topk_blocks(None, ctypes.byref(e), ctypes.byref(pr), None, None, None) == 0


def _dshape(**kw):
    d = dict(batch=2, q_len=1, kv_len=4096, q_start=0, num_q_heads=28, num_kv_heads=4, head_dim=128)
    d.update(kw)
    return nsa.make_shape(**d)


def _decode(shape, params=None, dtype=nsa.NSA_BF16, ws=1 << 40, kc=FAKE, table=None, max_pages=0, num_pages=0):
    L = nsa.lib()
    pr = params or _params(top_n=16, window=512)
    return L.nsa_decode_fwd(FAKE, FAKE, FAKE, kc, FAKE, FAKE, None, dtype, ctypes.byref(shape), ctypes.byref(pr),
                            FAKE, table, max_pages, num_pages, FAKE, None, None, None, None, FAKE, ws, None)


def test_decode_varlen_validates_first():
    pr = _params(top_n=16, window=512)
    need = nsa.nsa_decode_workspace_size(_dshape(), pr, nsa.NSA_BF16)
    assert need > 0
    assert nsa.nsa_decode_workspace_size(_dshape(), pr, nsa.NSA_F32) == 0
    assert _decode(_dshape(q_len=2)) == nsa.NSA_ERR_INVALID_ARG
    assert _decode(_dshape(), dtype=nsa.NSA_F32) == nsa.NSA_ERR_UNSUPPORTED
    assert _decode(_dshape(head_dim=64)) == nsa.NSA_ERR_UNSUPPORTED
    assert _decode(_dshape(kv_len=31)) == nsa.NSA_ERR_UNSUPPORTED          # no compressed block at capacity
    assert _decode(_dshape(), kc=None) == nsa.NSA_ERR_INVALID_ARG
    assert _decode(_dshape(), ws=need - 1) == nsa.NSA_ERR_WORKSPACE_TOO_SMALL
    # a page table must cover the capacity and name a non-empty pool
    assert _decode(_dshape(), table=FAKE, max_pages=63, num_pages=100) == nsa.NSA_ERR_INVALID_ARG
    assert _decode(_dshape(), table=FAKE, max_pages=64, num_pages=0) == nsa.NSA_ERR_INVALID_ARG
    assert "page" in nsa.last_error() or "num_pages" in nsa.last_error()
    assert _decode(_dshape(batch=0)) == nsa.NSA_OK                       # empty batch launches nothing


def test_decode_noalloc_validates_first():
    """The no-allocation decode rejects what nsa_decode_fwd rejects, and batches whose workspace
    exceeds the library's 64 MiB device scratch, before any launch."""
    L = nsa.lib()
    pr = _params(top_n=16, window=512)

    def call(shape, dtype=nsa.NSA_BF16, kc=FAKE):
        return L.nsa_decode_fwd_noalloc(FAKE, FAKE, FAKE, kc, FAKE, FAKE, None, dtype, ctypes.byref(shape),
                                        ctypes.byref(pr), FAKE, None, 0, 0, FAKE, None, None, None, None, None)

    assert call(_dshape(q_len=2)) == nsa.NSA_ERR_INVALID_ARG
    assert call(_dshape(), dtype=nsa.NSA_F32) == nsa.NSA_ERR_UNSUPPORTED
    assert call(_dshape(), kc=None) == nsa.NSA_ERR_INVALID_ARG
    big = _dshape(batch=64, kv_len=1 << 19)
    assert nsa.nsa_decode_workspace_size(big, pr, nsa.NSA_BF16) > 64 << 20
    assert call(big) == nsa.NSA_ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in nsa.last_error()
    assert nsa.nsa_decode_workspace_size(_dshape(batch=16, kv_len=65536), pr, nsa.NSA_BF16) < 64 << 20
    assert call(_dshape(batch=0)) == nsa.NSA_OK


def test_compress_append_validates_first():
    L = nsa.lib()

    def call(dtype=nsa.NSA_BF16, D=128, n_new=1, table=None, max_pages=0, num_pages=0, k=FAKE):
        return L.nsa_compress_append(k, FAKE, dtype, 2, 4096, 4, D, FAKE, FAKE, 32, 16, None, table, max_pages,
                                     num_pages, n_new, FAKE, FAKE, None)

    assert call(dtype=nsa.NSA_F32) == nsa.NSA_ERR_UNSUPPORTED
    assert call(dtype=5) == nsa.NSA_ERR_INVALID_ARG
    assert call(D=64) == nsa.NSA_ERR_UNSUPPORTED
    assert call(n_new=-1) == nsa.NSA_ERR_INVALID_ARG
    assert call(k=None) == nsa.NSA_ERR_INVALID_ARG
    assert call(table=FAKE, max_pages=10, num_pages=8) == nsa.NSA_ERR_INVALID_ARG
    assert call(n_new=0, k=None) == nsa.NSA_OK                            # nothing appended


def test_gate_proj_validates_first():
    L = nsa.lib()

    def call(dtype=nsa.NSA_BF16, hidden=3584, hq=28, x=FAKE, batch=1, seq=100):
        return L.nsa_gate_proj(x, FAKE, None, dtype, batch, seq, hidden, hq, FAKE, None)

    assert call(dtype=nsa.NSA_F32) == nsa.NSA_ERR_UNSUPPORTED
    assert call(dtype=3) == nsa.NSA_ERR_INVALID_ARG
    assert call(hidden=100) == nsa.NSA_ERR_UNSUPPORTED     # not a multiple of 64
    assert call(hq=33) == nsa.NSA_ERR_UNSUPPORTED          # more than 96 gate outputs
    assert call(hq=0) == nsa.NSA_ERR_INVALID_ARG
    assert call(x=None) == nsa.NSA_ERR_INVALID_ARG
    assert call(x=FAKE + 8) == nsa.NSA_ERR_INVALID_ARG     # misaligned
    assert call(x=None, seq=0) == nsa.NSA_OK               # no tokens: nothing launched


def test_branch_kv_decode_needs_one_selection_window_kv():
    L = nsa.lib()
    sh = _dshape(batch=2, q_len=1, kv_len=4096, q_start=4095)
    pr = _params(top_n=16, window=512)
    need = nsa.nsa_hybrid_layer_workspace_size(sh, pr, nsa.NSA_BF16)

    def call(kw):
        return L.nsa_hybrid_layer_fwd_branch_kv(FAKE, FAKE, FAKE, FAKE, FAKE, kw, FAKE, FAKE, FAKE, None, None, FAKE,
                                                None, nsa.NSA_BF16, ctypes.byref(sh), ctypes.byref(pr), FAKE, None,
                                                None, None, None, FAKE, need, None)

    assert call(FAKE + 4096) == nsa.NSA_ERR_UNSUPPORTED     # window keys differ from selection keys
    assert "selection and window" in nsa.last_error()
    sh2 = _dshape(batch=2, q_len=4096, kv_len=4096)
    assert L.nsa_hybrid_layer_fwd_branch_kv(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE,
                                            None, nsa.NSA_BF16, ctypes.byref(sh2), ctypes.byref(pr), FAKE, None, None,
                                            None, None, FAKE, 1 << 40, None) == nsa.NSA_ERR_INVALID_ARG


def test_backward_validates_first():
    L = nsa.lib()
    pr = _params()

    def call(sh, idx=FAKE, ws=1 << 40, dq=FAKE):
        return L.nsa_hybrid_layer_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, idx, FAKE, nsa.NSA_BF16,
                                      ctypes.byref(sh), ctypes.byref(pr), dq, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws,
                                      None)

    assert call(_shape(head_dim=72)) == nsa.NSA_ERR_UNSUPPORTED      # not a multiple of 64
    assert call(_shape(), idx=None) == nsa.NSA_ERR_INVALID_ARG        # the forward's chosen blocks are required
    assert call(_shape(), dq=None) == nsa.NSA_ERR_INVALID_ARG
    need = nsa.nsa_hybrid_layer_bwd_workspace_size(_shape(), pr, nsa.NSA_BF16)
    assert need > 0 and call(_shape(), ws=need - 1) == nsa.NSA_ERR_WORKSPACE_TOO_SMALL
    assert call(_shape(q_len=0)) == nsa.NSA_OK                        # no rows: nothing launched


def test_layer_workspace_rows():
    """Row chunks: at 128K the default workspace stays within 7 GiB (one pass needs about 19 GB) and
    is the size of a whole number of 16K-row chunks (32K rows), the size grows with the chunk, and a
    workspace below the 64-row size is refused before any launch."""
    sh = _dshape(batch=1, q_len=131072, kv_len=131072)
    pr = _params(top_n=16, window=512)
    bf = nsa.NSA_BF16
    full = nsa.nsa_hybrid_layer_workspace_size_rows(sh, pr, bf, 0)
    dflt = nsa.nsa_hybrid_layer_workspace_size(sh, pr, bf)
    assert full > 16 << 30 and 0 < dflt <= 7 << 30
    sizes = [nsa.nsa_hybrid_layer_workspace_size_rows(sh, pr, bf, r) for r in (64, 1000, 1024, 32768, 131072)]
    assert sizes[0] < sizes[2] < sizes[3] < sizes[4] == full
    assert sizes[1] == nsa.nsa_hybrid_layer_workspace_size_rows(sh, pr, bf, 960)   # chunks are multiples of 64
    assert dflt == sizes[3]  # the largest chunk within 7 GiB (43,712 rows), rounded down to 16K rows
    assert nsa.nsa_hybrid_layer_workspace_size_rows(sh, pr, bf, -1) == 0
    L = nsa.lib()
    st = L.nsa_hybrid_layer_fwd(FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, bf, ctypes.byref(sh),
                                ctypes.byref(pr), FAKE, None, None, None, None, FAKE, sizes[0] - 1, None)
    assert st == nsa.NSA_ERR_WORKSPACE_TOO_SMALL and "workspace" in nsa.last_error()
    # the generic path and decode run in one pass: their sizes do not depend on the chunk
    f32 = nsa.NSA_F32
    small = _dshape(batch=1, q_len=4096, kv_len=4096)
    assert (nsa.nsa_hybrid_layer_workspace_size_rows(small, pr, f32, 64) ==
            nsa.nsa_hybrid_layer_workspace_size_rows(small, pr, f32, 0))
    dec = _dshape(batch=4, q_len=1, kv_len=8192, q_start=8191)
    assert (nsa.nsa_hybrid_layer_workspace_size_rows(dec, pr, bf, 64) ==
            nsa.nsa_hybrid_layer_workspace_size(dec, pr, bf))


@pytest.mark.parametrize("T,B,q0,rows,ls", [(131072, 1, 0, 40960, 64), (131072, 1, 0, 1024, 64),
                                            (36352, 2, 0, 4096, 64), (9000, 1, 0, 1024, 64),
                                            (70000, 1, 5000, 8192, 64), (131072, 1, 0, 8192, 32),
                                            (131072, 1, 0, 16384, 128), (20000, 2, 3000, 2048, 32)])
def test_layer_chunk_workspace_covers_every_chunk(T, B, q0, rows, ls):
    """The chunked workspace must hold what every chunk needs as a call of its own (rows placed where
    the chunk sits: scratch such as the key splits of long text rows grows with the position)."""
    pr = _params(top_n=16, window=512, sel_block=ls)
    bf = nsa.NSA_BF16
    sh = _dshape(batch=B, q_len=T - q0, kv_len=T, q_start=q0)
    carve = nsa.nsa_hybrid_layer_workspace_size_rows(sh, pr, bf, rows)
    for r0 in range(0, T - q0, rows):
        n = min(rows, T - q0 - r0)
        one = _dshape(batch=1, q_len=n, kv_len=T, q_start=q0 + r0)
        assert nsa.nsa_hybrid_layer_workspace_size_rows(one, pr, bf, 0) <= carve, (r0, n)
