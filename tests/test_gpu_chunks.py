"""Row chunks of the layer: a prefill run as passes over chunks of query rows (workspace sized for
at most rows_per_chunk rows) must give bitwise the same outputs and chosen blocks as one pass, since
every stage except the K / V compression is independent across rows.  Cases: two sequences with
ragged ends and text rows at both ends (chunks of 1024 rows, the last one partial), a block of query
rows that starts inside the sequence, 8 query heads per KV head (the other compression-branch
kernel), text rows deep enough in the sequence that their dense pass splits the keys (scratch that
grows with the chunk's position), the per-branch K / V entry point, and the phase timing of a chunked
call."""
import numpy as np
import pytest

from gpu_util import flush, host
from sparse_attention_long_fwd_amd import nsa, synth
from test_gpu_parity import _branch_inputs, _wl, run_layer, run_layer_branch_kv

pytestmark = pytest.mark.gpu
DEV = "cuda"
OUTS = ("out", "o_cmp", "o_slc", "o_swa", "idx")


def _same(a, b):
    for name in OUTS:
        assert np.array_equal(host(a[name]), host(b[name])), name


@pytest.mark.parametrize("case", ["batch2-ragged", "query-block", "g8", "text-splits"])
def test_layer_chunks_bitwise(case):
    if case == "batch2-ragged":
        wl = _wl(T=5000 + 37, B=2, lead=64, tail=29, n=16, w=512)
    elif case == "text-splits":  # text rows past 8192 tokens: their dense pass splits the keys
        wl = _wl(T=9000, lead=64, tail=120, n=16, w=512)
    elif case == "query-block":  # rows 1000 .. 5999 of a 6000-token sequence
        wl = _wl(T=6000, q_start=1000, lead=0, tail=40, n=16, w=512)
    else:
        wl = _wl(T=3000, Hq=16, Hkv=2, lead=64, tail=30, n=8, w=256)
    flush("layer chunks %s" % case)
    inp = synth.make_inputs(wl, DEV)
    one = run_layer(wl, inp, rows_per_chunk=0)
    for rows in (1024, 640):
        _same(run_layer(wl, inp, rows_per_chunk=rows), one)


def test_layer_chunks_branch_kv():
    wl = _wl(T=4000 + 11, B=2, lead=32, tail=16, n=16, w=512)
    flush("layer chunks branch-kv")
    inp = _branch_inputs(wl)
    _same(run_layer_branch_kv(wl, inp, rows_per_chunk=1024), run_layer_branch_kv(wl, inp, rows_per_chunk=0))


def test_layer_chunks_phase_timing():
    wl = _wl(T=4096, lead=64, tail=64, n=16, w=512)
    inp = synth.make_inputs(wl, DEV)
    run_layer(wl, inp, rows_per_chunk=1024)
    nsa.profile_enable(True)
    try:
        run_layer(wl, inp, rows_per_chunk=1024)
        ph = nsa.profile_read()
    finally:
        nsa.profile_enable(False)
    flush("  phases over 4 chunks (ms): %s" % ph)
    assert len(ph) == 5 and min(ph) >= 0.0 and ph[1] > 0.0 and ph[4] > 0.0
