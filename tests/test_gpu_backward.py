"""GPU parity of the backward pass (nsa_hybrid_layer_bwd) against the fp64 oracle's
backward, through the C ABI.  The chosen blocks come from the oracle's forward and feed
both sides (selection passes no gradient).

Tolerance (fp32 accumulation on both fp32 and bf16 inputs, which widen exactly): per
output, max-abs error <= 1e-4 x max|reference| + 1e-5; the compression weight gradients
sum over every (block, KV head, channel) and get 3e-4 x max|reference| + 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import flush, host
from sparse_attention_long_fwd_amd import nsa, synth
from test_gpu_parity import _wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL = {"dq": 1e-4, "dk": 1e-4, "dv": 1e-4, "dgates": 1e-4, "dw_k": 3e-4, "dw_v": 3e-4}
KEYS = {"dq": "dq", "dk": "dk", "dv": "dv", "dgates": "d_gates", "dw_k": "dw_k", "dw_v": "dw_v"}


def _setup(wl, seed_dout=900):
    inp = synth.make_inputs(wl, DEV)
    B, Tq, Hq, D = inp["q"].shape
    dout = synth.normal(1000 * wl.index + seed_dout, (B, Tq, Hq, D), DEV).to(wl.torch_dtype)
    idx = torch.full((B, Tq, wl.num_kv_heads, wl.top_n), -1, dtype=torch.int32)
    for b in range(B):
        res = oracle.layer(host(inp["q"][b]), host(inp["k"][b]), host(inp["v"][b]), host(inp["w_k"]),
                           host(inp["w_v"]), host(inp["gates"][b]), host(inp["is_video"][b]), wl.params(),
                           q_start=wl.q_start)
        idx[b] = torch.from_numpy(res["idx"])
    return inp, dout, idx.to(DEV)


def _run(wl, inp, dout, idx):
    q = inp["q"]
    B, Tq, Hq, D = q.shape
    sh = nsa.make_shape(B, Tq, wl.kv_len, wl.q_start, Hq, wl.num_kv_heads, D)
    pr = nsa.make_params(**wl.params())
    g = nsa.nsa_hybrid_layer_bwd(q, inp["k"], inp["v"], inp["gates"], idx, dout, sh, pr, w_k=inp["w_k"],
                                 w_v=inp["w_v"], is_video=inp["is_video"])
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("case", ["f32-tiny", "bf16-ragged", "bf16-batch2", "bf16-short", "bf16-no-cmp-block",
                                  "bf16-all-text", "bf16-q-start", "bf16-row-chunks"])
def test_layer_backward(case):
    if case == "f32-tiny":
        wl = _wl(dtype="f32", T=300, Hq=4, Hkv=1, D=64, n=4, w=128, lead=16, corr=False)
    elif case == "bf16-ragged":
        wl = _wl(T=1037, Hq=14, Hkv=2, lead=64, tail=13, n=6, w=100)
    elif case == "bf16-batch2":
        wl = _wl(T=700, B=2, lead=40, n=8, w=256)
    elif case == "bf16-short":
        wl = _wl(T=70, Hq=8, Hkv=2, n=4, w=64)
    elif case == "bf16-no-cmp-block":
        wl = _wl(T=31, Hq=8, Hkv=2, n=4, w=16)
    elif case == "bf16-all-text":
        wl = _wl(T=200, Hq=8, Hkv=2, lead=200, n=4, w=64)
    elif case == "bf16-q-start":  # a block of query rows at the end of the sequence
        wl = _wl(T=900, Hq=14, Hkv=2, q_start=600, q_len=300, lead=0, tail=20, n=6, w=128)
    else:  # enough rows that the key kernels split them into several chunks (3 and 5)
        wl = _wl(T=4500, Hq=8, Hkv=2, lead=32, tail=40, n=6, w=200)
    flush("backward %s" % case)
    inp, dout, idx = _setup(wl)
    got = _run(wl, inp, dout, idx)
    stats = {}
    tot = {"dk": 0.0, "dv": 0.0}
    for b in range(wl.batch):
        ref = oracle.layer_bwd(host(inp["q"][b]), host(inp["k"][b]), host(inp["v"][b]), host(inp["w_k"]),
                               host(inp["w_v"]), host(inp["gates"][b]), host(inp["is_video"][b]), wl.params(),
                               host(dout[b]), q_start=wl.q_start, idx=host(idx[b]))
        for key in ("dq", "dk", "dv", "dgates"):
            r, g = ref[key], host(got[KEYS[key]][b]).astype(np.float64)
            err = float(np.abs(g - r).max())
            lim = REL[key] * float(np.abs(r).max()) + 1e-5
            stats["%s[%d]" % (key, b)] = (err, lim)
            assert err <= lim, (key, b, err, lim)
        if b == 0:
            dw = {"dw_k": ref["dw_k"], "dw_v": ref["dw_v"]}
        else:
            dw = {key: dw[key] + ref[key] for key in dw}
    for key in ("dw_k", "dw_v"):
        g = host(got[KEYS[key]]).astype(np.float64)
        err = float(np.abs(g - dw[key]).max())
        lim = REL[key] * float(np.abs(dw[key]).max()) + 1e-5
        stats[key] = (err, lim)
        assert err <= lim, (key, err, lim)
    flush("  %s" % {k: "%.2e/%.2e" % v for k, v in stats.items()})
