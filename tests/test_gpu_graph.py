"""HIP-graph capture of the library's calls: each captured sequence is replayed several
times, with eager work of the program and synchronisations between the replays, and every
replay must reproduce the eager result bit for bit (the kernels are deterministic, and no
call records a memset node)."""
import numpy as np
import pytest
import torch

from gpu_util import flush
from sparse_attention_long_fwd_amd import nsa, synth
from test_gpu_parity import _wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _replays(capture_fn, outputs, eager_noise, n=3):
    """Capture capture_fn on a side stream, replay n times; return the outputs of each replay."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            capture_fn(side)
    torch.cuda.current_stream().wait_stream(side)
    res = []
    for i in range(n):
        for o in outputs:
            _sentinel(o)  # stale values must not survive; entries a call leaves untouched stay equal
        eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        res.append([o.clone() for o in outputs])
    return res


def _sentinel(o):
    o.fill_(1234.5 if o.is_floating_point() else -7)


def _noise():
    a = torch.randn(1 << 20, device=DEV)
    (a * 2 + 1).sum().item()


def test_graph_decode_layer():
    wl = _wl(T=5000, B=3, q_start=4999, q_len=1, lead=0, tail=0)
    flush("graph decode layer")
    inp = synth.make_inputs(wl, DEV)
    inp["is_video"][1] = 0
    kc, vc = nsa.nsa_compress_kv(inp["k"], inp["v"], inp["w_k"], inp["w_v"])
    q = inp["q"]
    B, Tq, Hq, D = q.shape
    sh = nsa.make_shape(B, Tq, wl.kv_len, wl.q_start, Hq, 4, D)
    pr = nsa.make_params(**wl.params())
    ws = torch.empty(nsa.nsa_hybrid_layer_workspace_size(sh, pr, nsa.NSA_BF16), dtype=torch.uint8, device=DEV)
    out, o_slc = torch.empty_like(q), torch.empty_like(q)
    idx = torch.empty(B, Tq, 4, wl.top_n, dtype=torch.int32, device=DEV)

    def call(stream):
        nsa.nsa_hybrid_layer_fwd(q, inp["k"], inp["v"], inp["gates"], sh, pr, k_cmp_in=kc, v_cmp_in=vc,
                                 is_video=inp["is_video"], out=out, o_slc=o_slc, block_idx_out=idx, workspace=ws,
                                 stream=stream)

    for o in (out, o_slc, idx):
        _sentinel(o)
    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [out.clone(), o_slc.clone(), idx.clone()]
    for r in _replays(call, [out, o_slc, idx], _noise):
        for a, b in zip(r, ref):
            assert torch.equal(a, b)


def test_graph_prefill_layer():
    wl = _wl(T=4096, lead=256, tail=256)
    flush("graph prefill layer")
    inp = synth.make_inputs(wl, DEV)
    q = inp["q"]
    B, Tq, Hq, D = q.shape
    sh = nsa.make_shape(B, Tq, wl.kv_len, 0, Hq, 4, D)
    pr = nsa.make_params(**wl.params())
    ws = torch.empty(nsa.nsa_hybrid_layer_workspace_size(sh, pr, nsa.NSA_BF16), dtype=torch.uint8, device=DEV)
    out, o_cmp = torch.empty_like(q), torch.empty_like(q)

    def call(stream):
        nsa.nsa_hybrid_layer_fwd(q, inp["k"], inp["v"], inp["gates"], sh, pr, w_k=inp["w_k"], w_v=inp["w_v"],
                                 is_video=inp["is_video"], out=out, o_cmp=o_cmp, workspace=ws, stream=stream)

    for o in (out, o_cmp):
        _sentinel(o)
    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [out.clone(), o_cmp.clone()]
    for r in _replays(call, [out, o_cmp], _noise):
        for a, b in zip(r, ref):
            assert torch.equal(a, b)


def test_graph_varlen_decode_step():
    """Compressed-cache append for one token plus the variable-length paged decode."""
    lens = [4097, 33, 1000, 2500]
    cap = 4160
    wl = _wl(T=cap, B=len(lens), q_start=cap - 1, q_len=1)
    flush("graph varlen decode")
    inp = synth.make_inputs(wl, DEV)
    B, Hkv, D = len(lens), 4, 128
    mp = cap // 64
    perm = torch.from_numpy(np.random.default_rng(3).permutation(B * mp)).to(DEV)
    kp = torch.empty(B * mp, 64, Hkv, D, dtype=torch.bfloat16, device=DEV)
    vp = torch.empty_like(kp)
    kp[perm] = inp["k"].view(B * mp, 64, Hkv, D)
    vp[perm] = inp["v"].view(B * mp, 64, Hkv, D)
    table = perm.view(B, mp).to(torch.int32)
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    nc = (cap - 32) // 16 + 1
    kc = torch.zeros(B, nc, Hkv, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    nsa.nsa_compress_append(kp, vp, inp["w_k"], inp["w_v"], kc, vc, cap, cap, kv_lens=lt, page_table=table)
    q = inp["q"]
    sh = nsa.make_shape(B, 1, cap, 0, q.shape[2], Hkv, D)
    pr = nsa.make_params(**wl.params())
    ws = torch.empty(nsa.nsa_decode_workspace_size(sh, pr, nsa.NSA_BF16), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(q)

    def call(stream):
        nsa.nsa_compress_append(kp, vp, inp["w_k"], inp["w_v"], kc, vc, cap, 1, kv_lens=lt, page_table=table,
                                stream=stream)
        nsa.nsa_decode_fwd(q, kp, vp, kc, vc, inp["gates"], sh, pr, kv_lens=lt, page_table=table,
                           is_video=inp["is_video"], out=out, workspace=ws, stream=stream)

    _sentinel(out)
    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [out.clone(), kc.clone()]
    for r in _replays(call, [out], _noise):
        assert torch.equal(r[0], ref[0])
    assert torch.equal(kc, ref[1])
