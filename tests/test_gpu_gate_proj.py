"""GPU parity of the gate projection (hidden states -> per-head branch gates) against
the fp64 oracle, through the C ABI: ragged token counts, gate counts that are and are
not multiples of 4, with and without bias, the 128K Qwen2.5-VL-7B shape on sampled
rows, and the gates fed into the layer.

Tolerance: gates max-abs 2e-5 (fp32 accumulation of up to 3584 bf16 products, the
logistic's slope is at most 1/4); layer outputs as in the other parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, flush, host, maxabs
from sparse_attention_long_fwd_amd import nsa, synth
from test_gpu_parity import _wl, compare_layer, run_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"
GTOL = 2e-5


@pytest.mark.parametrize("B,T,hidden,Hq,bias", [(2, 300, 3584, 28, True), (1, 1, 192, 5, True),
                                                (1, 1000, 1024, 32, False), (3, 129, 64, 1, True)])
def test_gate_proj(B, T, hidden, Hq, bias):
    flush("gate_proj B=%d T=%d hidden=%d Hq=%d bias=%s" % (B, T, hidden, Hq, bias))
    wl = _wl(T=T, B=B, Hq=Hq, Hkv=1)
    gi = synth.make_gate_inputs(wl, DEV, hidden=hidden)
    bg = gi["b_g"] if bias else None
    g = nsa.nsa_gate_proj(gi["x"], gi["w_g"], bg)
    torch.cuda.synchronize()
    assert g.shape == (B, T, Hq, 3)
    for b in range(B):
        ref = oracle.gate_proj(host(gi["x"][b]), host(gi["w_g"]), None if bg is None else host(bg))
        assert maxabs(host(g[b]).reshape(T, 3 * Hq), ref) <= GTOL


def test_gate_proj_full_size_sampled():
    wl = synth.WORKLOADS["128k"]
    flush("gate_proj 128k")
    gi = synth.make_gate_inputs(wl, DEV)
    g = nsa.nsa_gate_proj(gi["x"], gi["w_g"], gi["b_g"])
    torch.cuda.synchronize()
    T = wl.q_len
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([np.arange(128), np.arange(T - 128, T), rng.choice(T, 1500, replace=False)]))
    ri = torch.from_numpy(rows).to(DEV)
    ref = oracle.gate_proj(host(gi["x"][0][ri]), host(gi["w_g"]), host(gi["b_g"]))
    assert maxabs(host(g[0][ri]).reshape(len(rows), -1), ref) <= GTOL


def test_gates_from_hidden_states_into_layer():
    wl = _wl(T=1024, lead=64, tail=32, n=8, w=256)
    flush("gate_proj -> layer T=%d" % wl.kv_len)
    inp = synth.make_inputs(wl, DEV)
    gi = synth.make_gate_inputs(wl, DEV)
    inp["gates"] = nsa.nsa_gate_proj(gi["x"], gi["w_g"], gi["b_g"])
    got = run_layer(wl, inp)
    ref_g = oracle.gate_proj(host(gi["x"][0]), host(gi["w_g"]), host(gi["b_g"]))
    assert maxabs(host(inp["gates"][0]).reshape(wl.q_len, -1), ref_g) <= GTOL
    # the oracle layer on the oracle's gates (fp64, rounded to fp32 as the layer's gate input is)
    inp_ref = dict(inp)
    inp_ref["gates"] = torch.from_numpy(ref_g.reshape(1, wl.q_len, -1, 3).astype(np.float32)).to(DEV)
    compare_layer(wl, inp_ref, got, np.arange(wl.q_len))
