"""GPU parity of the layer at selection blocks of 32 and 128 tokens (the l' axis), against the fp64
oracle through the C ABI, with the rules of the other parity tests (chosen blocks identical where
the oracle's gap exceeds 1e-3, outputs within 2e-2).

With 4..7 query heads per KV head the MFMA path serves these sizes: the group kernel forms the
importance of 32-token blocks (two per lane, each half of the straddling compressed keys at its
ends) or of 128-token blocks (one per lane pair, joined with one lane exchange), and the selection
kernel stages 32- or 128-token key tiles.  With 8 heads per KV head, and for compressed keys that
the caller passes in, the compression branch runs on the generic kernel; those cases are covered
here too.  Cases: ragged ends, two sequences, text rows at both ends, query blocks at aligned and
unaligned positions, one query row, and the two 128K budget points (32 n + w and 128 n + w at 1536
tokens) on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import flush, host
from sparse_attention_long_fwd_amd import synth
from test_gpu_parity import _sample_rows, _wl, compare_layer, run_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = {
    # ls, workload
    "ls32-g7-ragged": lambda: _wl(T=6000 + 13, Hq=28, Hkv=4, lead=64, tail=20, n=16, w=512, sel_block=32),
    "ls128-g4-batch2": lambda: _wl(T=9000 + 37, B=2, Hq=8, Hkv=2, lead=0, tail=40, n=8, w=512, sel_block=128),
    "ls32-g6-query-block": lambda: _wl(T=5100, Hq=12, Hkv=2, q_start=4100, lead=0, tail=17, n=12, w=256,
                                       sel_block=32),
    "ls128-g5-query-block": lambda: _wl(T=7000, Hq=10, Hkv=2, q_start=6016, lead=0, tail=9, n=6, w=384,
                                        sel_block=128),
    "ls32-g8-generic": lambda: _wl(T=3000, Hq=16, Hkv=2, lead=64, tail=30, n=8, w=256, sel_block=32),
    "ls128-g4-one-row": lambda: _wl(T=5000, Hq=8, Hkv=2, q_start=4999, lead=0, tail=0, n=8, w=256,
                                    sel_block=128),
}


def _rows(wl, step, seed):
    rng = np.random.default_rng(seed)
    T = wl.q_len
    rows = set(range(int(rng.integers(0, step)), T, step))
    rows |= set(range(min(40, T))) | set(range(max(0, T - 40), T))
    # the first rows past 1024-token key tiles (where the importance carries across tiles)
    for edge in (1024, 2048, 4096):
        e = edge - wl.q_start
        rows |= set(range(max(0, e - 20), min(T, e + 20)))
    return np.array(sorted(r for r in rows if 0 <= r < T), dtype=np.int64)


@pytest.mark.parametrize("case", list(CASES))
def test_layer_sel_block(case):
    wl = CASES[case]()
    flush("selection block %d: %s" % (wl.sel_block, case))
    inp = synth.make_inputs(wl, DEV)
    got = run_layer(wl, inp)
    for b in range(wl.batch):
        rows = _rows(wl, 9, b)
        flush("  batch %d: %d rows" % (b, len(rows)))
        compare_layer(wl, inp, got, rows, b)


@pytest.mark.parametrize("ls", [32, 128])
def test_layer_sel_block_generic_path(ls):
    """The same layer on the generic kernels (nsa_set_force_generic) against the oracle."""
    from sparse_attention_long_fwd_amd import nsa
    wl = _wl(T=2500 + 7, Hq=14, Hkv=2, lead=32, tail=11, n=8, w=256, sel_block=ls)
    flush("selection block %d generic path" % ls)
    inp = synth.make_inputs(wl, DEV)
    prev = nsa.set_force_generic(True)
    try:
        got = run_layer(wl, inp)
    finally:
        nsa.set_force_generic(prev)
    compare_layer(wl, inp, got, _rows(wl, 7, 1))


@pytest.mark.parametrize("ls", [32, 128])
def test_layer_sel_block_compressed_in(ls):
    """Compressed keys / values from the caller (here the oracle's, rounded to bf16): the compression
    branch then runs on the generic kernel and the combine reads its bf16 output."""
    wl = _wl(T=4000 + 21, Hq=28, Hkv=4, lead=64, tail=20, n=12, w=512, sel_block=ls)
    flush("selection block %d, caller's compressed K/V" % ls)
    inp = synth.make_inputs(wl, DEV)
    kc = oracle.compress(host(inp["k"][0]), host(inp["w_k"]), 32, 16)
    vc = oracle.compress(host(inp["v"][0]), host(inp["w_v"]), 32, 16)
    kct = torch.from_numpy(kc[None]).to(DEV).to(torch.bfloat16)
    vct = torch.from_numpy(vc[None]).to(DEV).to(torch.bfloat16)
    got = run_layer(wl, inp, k_cmp_in=kct, v_cmp_in=vct)
    compare_layer(wl, inp, got, _rows(wl, 9, 2), 0, kc=host(kct[0]).astype(np.float64),
                  vc=host(vct[0]).astype(np.float64))


@pytest.mark.parametrize("ls,n,w", [(32, 32, 512), (128, 8, 512)])
def test_layer_sel_block_128k_sampled(ls, n, w):
    """The 128K workload at a 1536-token budget (ls n + w) with 32- and 128-token blocks."""
    wl = synth.WORKLOADS["128k"].with_(sel_block=ls, top_n=n, window=w)
    flush("128K selection block %d n=%d w=%d" % (ls, n, w))
    inp = synth.make_inputs(wl, DEV)
    got = run_layer(wl, inp)
    rows = _sample_rows(wl, seed=ls, text=4, edge=16)[::3]
    flush("  %d sampled rows" % len(rows))
    compare_layer(wl, inp, got, rows)
