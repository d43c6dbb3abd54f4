"""GPU parity of the variable-length / paged decode step and of the incremental
compressed-cache update, through the C ABI, against the fp64 oracle run on each
sequence's own tokens (a contiguous copy of its first L_b rows).

Lengths cover: a single token, fewer tokens than one compressed block, exactly
one block, non-multiples of the compression stride, whole selection blocks, a
text row, and the capacity itself.  Tolerances and the index rule are those of
the other parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, flush, host, maxabs
from sparse_attention_long_fwd_amd import nsa, synth
from test_gpu_parity import _wl, compare_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"
PAGE = nsa.PAGE_ROWS
LENS = [5000, 1, 20, 32, 1013, 576, 4097, 5120]
CAP = 5120


def _ncmp(L):
    return 0 if L < 32 else (L - 32) // 16 + 1


def _paged(x, lens, seed, extra=5):
    """Page pool [num_pages, 64, H, D] holding x[b, :L_b] at seeded page ids; table [B, max_pages]."""
    B, T, H, D = x.shape
    mp = (T + PAGE - 1) // PAGE
    n = B * mp + extra
    perm = np.random.default_rng(seed).permutation(n)
    pool = torch.zeros(n, PAGE, H, D, dtype=x.dtype, device=x.device)
    table = np.full((B, mp), -1, dtype=np.int32)
    for b, L in enumerate(lens):
        for i in range((L + PAGE - 1) // PAGE):
            pid = int(perm[b * mp + i])
            table[b, i] = pid
            r = x[b, i * PAGE:(i + 1) * PAGE]
            pool[pid, :r.shape[0]] = r
    return pool, torch.from_numpy(table).to(x.device)


def _inputs(lens, text=(3,), seed_index=11):
    wl = _wl(T=CAP, B=len(lens), q_start=CAP - 1, q_len=1).with_(index=seed_index)
    inp = synth.make_inputs(wl, DEV)
    for b in text:
        inp["is_video"][b] = 0
    return wl, inp


def _decode(wl, inp, kc, vc, lens, k=None, v=None, table=None):
    q = inp["q"]
    B, _, Hq, D = q.shape
    Hkv = inp["k"].shape[2]
    sh = nsa.make_shape(B, 1, CAP, 0, Hq, Hkv, D)
    pr = nsa.make_params(**wl.params())
    o_cmp, o_slc, o_swa = torch.zeros_like(q), torch.zeros_like(q), torch.zeros_like(q)
    idx = torch.full((B, 1, Hkv, wl.top_n), -1, dtype=torch.int32, device=DEV)
    kv_lens = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = nsa.nsa_decode_fwd(q, inp["k"] if k is None else k, inp["v"] if v is None else v, kc, vc, inp["gates"],
                             sh, pr, kv_lens=kv_lens, page_table=table, is_video=inp["is_video"], o_cmp=o_cmp,
                             o_slc=o_slc, o_swa=o_swa, block_idx_out=idx)
    torch.cuda.synchronize()
    return dict(out=out, o_cmp=o_cmp, o_slc=o_slc, o_swa=o_swa, idx=idx)


def _compare_each(wl, inp, got, kc, vc, lens):
    for b, L in enumerate(lens):
        wl_b = wl.with_(kv_len=L, q_start=L - 1, batch=1)
        inp_b = dict(q=inp["q"][b:b + 1], k=inp["k"][b:b + 1, :L], v=inp["v"][b:b + 1, :L],
                     gates=inp["gates"][b:b + 1], is_video=inp["is_video"][b:b + 1], w_k=inp["w_k"], w_v=inp["w_v"])
        got_b = {key: t[b:b + 1] for key, t in got.items()}
        nc = _ncmp(L)
        flush("  seq %d L=%d video=%d" % (b, L, int(inp["is_video"][b, 0])))
        compare_layer(wl_b, inp_b, got_b, np.arange(1), 0, kc=host(kc[b, :nc]).astype(np.float64),
                      vc=host(vc[b, :nc]).astype(np.float64))


def _oracle_cache(inp, lens, cap):
    """The compressed cache of each sequence's own tokens, from the oracle, rounded to bf16
    (blocks past a sequence's length stay 0); it feeds both sides."""
    B = len(lens)
    nc = _ncmp(cap)
    kc = np.zeros((B, nc, 4, 128), np.float32)
    vc = np.zeros_like(kc)
    for b, L in enumerate(lens):
        m = _ncmp(L)
        if m:
            kc[b, :m] = oracle.compress(host(inp["k"][b, :L]), host(inp["w_k"]), 32, 16)
            vc[b, :m] = oracle.compress(host(inp["v"][b, :L]), host(inp["w_v"]), 32, 16)
    return (torch.from_numpy(kc).to(DEV).to(torch.bfloat16), torch.from_numpy(vc).to(DEV).to(torch.bfloat16))


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_decode_varlen(layout):
    flush("decode varlen %s lens=%s" % (layout, LENS))
    wl, inp = _inputs(LENS)
    kc, vc = _oracle_cache(inp, LENS, CAP)
    if layout == "contiguous":
        got = _decode(wl, inp, kc, vc, LENS)
    else:
        kp, table = _paged(inp["k"], LENS, seed=1)
        vp, _ = _paged(inp["v"], LENS, seed=1)
        got = _decode(wl, inp, kc, vc, LENS, k=kp, v=vp, table=table)
    _compare_each(wl, inp, got, kc, vc, LENS)


def test_decode_varlen_full_size():
    """The bench's batch: 16 sequences of seeded lengths in [4096, 65536], 64K capacity, pages at
    shuffled pool positions; every sequence's row checked."""
    wlv = synth.WORKLOADS["decode_varlen"]
    lens = synth.decode_lengths(wlv)
    flush("decode varlen full size lens=%s" % lens)
    inp = synth.make_inputs(wlv, DEV)
    kc, vc = _oracle_cache(inp, lens, wlv.kv_len)
    kp, table = _paged(inp["k"], lens, seed=6)
    vp, _ = _paged(inp["v"], lens, seed=6)
    q = inp["q"]
    B, _, Hq, D = q.shape
    sh = nsa.make_shape(B, 1, wlv.kv_len, 0, Hq, 4, D)
    pr = nsa.make_params(**wlv.params())
    o_cmp, o_slc, o_swa = torch.zeros_like(q), torch.zeros_like(q), torch.zeros_like(q)
    idx = torch.full((B, 1, 4, wlv.top_n), -1, dtype=torch.int32, device=DEV)
    out = nsa.nsa_decode_fwd(q, kp, vp, kc, vc, inp["gates"], sh, pr,
                             kv_lens=torch.tensor(lens, dtype=torch.int32, device=DEV), page_table=table,
                             is_video=inp["is_video"], o_cmp=o_cmp, o_slc=o_slc, o_swa=o_swa, block_idx_out=idx)
    torch.cuda.synchronize()
    got = dict(out=out, o_cmp=o_cmp, o_slc=o_slc, o_swa=o_swa, idx=idx)
    _compare_each(wlv, inp, got, kc, vc, lens)


def test_decode_varlen_full_lengths_match_uniform_decode():
    """Every sequence at the capacity: the same kernels and the same bits as the layer's decode."""
    lens = [CAP] * 3
    wl, inp = _inputs(lens, text=(1,))
    kc, vc = _oracle_cache(inp, lens, CAP)
    a = _decode(wl, inp, kc, vc, lens)
    b = _decode(wl, inp, kc, vc, None)
    q = inp["q"]
    sh = nsa.make_shape(3, 1, CAP, CAP - 1, q.shape[2], 4, 128)
    pr = nsa.make_params(**wl.params())
    out = nsa.nsa_hybrid_layer_fwd(q, inp["k"], inp["v"], inp["gates"], sh, pr, k_cmp_in=kc, v_cmp_in=vc,
                                   is_video=inp["is_video"])
    torch.cuda.synchronize()
    for key in ("out", "o_cmp", "o_slc", "o_swa", "idx"):
        assert torch.equal(a[key], b[key]), key
    assert torch.equal(a["out"], out)


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_compress_append_stream(layout):
    """A decode stream: appends of 40, 1, 1, 15, 16, 17, 100, 1 and 300 tokens to every sequence;
    after each, the blocks complete within L_b equal a full compression of the first L_b tokens
    (bit for bit, the same sums and rounding) and the oracle's (bf16 rounding); the rest stay 0."""
    B, H, D, cap = 3, 4, 128, 1024
    wl = _wl(T=cap, B=B, Hq=28, Hkv=H)
    inp = synth.make_inputs(wl, DEV)
    k, v = inp["k"], inp["v"]
    full_k, full_v = nsa.nsa_compress_kv(k, v, inp["w_k"], inp["w_v"])
    nc = _ncmp(cap)
    kc = torch.zeros(B, nc, H, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    lens = np.array([0, 5, 40])
    if layout == "paged":
        kp, table = _paged(k, [cap] * B, seed=2)
        vp, _ = _paged(v, [cap] * B, seed=2)
    else:
        kp, vp, table = k, v, None
    for step, n_new in enumerate([40, 1, 1, 15, 16, 17, 100, 1, 300]):
        lens = np.minimum(lens + n_new, cap) if step else lens
        lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
        nsa.nsa_compress_append(kp, vp, inp["w_k"], inp["w_v"], kc, vc, cap, n_new, kv_lens=lt, page_table=table)
        torch.cuda.synchronize()
        for b in range(B):
            m = _ncmp(int(lens[b]))
            assert torch.equal(kc[b, :m], full_k[b, :m]) and torch.equal(vc[b, :m], full_v[b, :m]), (step, b)
            assert not kc[b, m:].any() and not vc[b, m:].any(), (step, b)
    flush("append %s final lens %s" % (layout, lens.tolist()))
    for b in range(B):
        L = int(lens[b])
        rk = oracle.compress(host(k[b, :L]), host(inp["w_k"]), 32, 16)
        rv = oracle.compress(host(v[b, :L]), host(inp["w_v"]), 32, 16)
        m = rk.shape[0]
        assert maxabs(host(kc[b, :m]), rk) <= TOL["bf16"] and maxabs(host(vc[b, :m]), rv) <= TOL["bf16"]
