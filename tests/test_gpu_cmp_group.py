"""GPU parity of the layer where the compression branch runs on the group kernel (4..7 query heads
per KV head; one wave per 16 rows x all heads of the group), against the fp64 oracle through the C
ABI, with the same rules as the other parity tests (chosen blocks identical where the oracle's gap
exceeds 1e-3, outputs within 2e-2).  Cases: 4, 6 and 7 query heads per KV head, two sequences,
ragged ends, text rows at both ends, a block of query rows starting at an unaligned position, and
value tiles whose magnitudes need the per-tile fp16 range scale."""
import numpy as np
import pytest

from gpu_util import flush
from sparse_attention_long_fwd_amd import synth
from test_gpu_parity import _wl, compare_layer, run_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rows(wl, lo, step, seed):
    """Every `step`-th row from `lo` (seeded offset), the rows around 4.1K and 8.2K tokens (where
    earlier kernels switched variants), and the first and last rows."""
    rng = np.random.default_rng(seed)
    T = wl.q_len
    rows = set(range(lo + int(rng.integers(0, step)), T, step))
    for edge in (4096, 4111, 4160, 8192, 8207, 8256):
        e = edge - wl.q_start
        rows |= set(range(max(0, e - 40), min(T, e + 40)))
    rows |= set(range(min(16, T))) | set(range(max(0, T - 48), T))
    return np.array(sorted(r for r in rows if 0 <= r < T), dtype=np.int64)


@pytest.mark.parametrize("case", ["g7-batch2-ragged", "g4", "g6-query-block"])
def test_layer_group_kernel(case):
    if case == "g7-batch2-ragged":
        wl = _wl(T=10000 + 37, B=2, Hq=28, Hkv=4, lead=64, tail=29, n=16, w=512)
        step = 11
    elif case == "g4":
        wl = _wl(T=9000, Hq=8, Hkv=2, lead=0, tail=40, n=8, w=256)
        step = 5
    else:  # query rows 8200 .. 9099 of a 9100-token sequence (chunked prefill), 6 heads per KV head
        wl = _wl(T=9100, Hq=12, Hkv=2, q_start=8200, lead=0, tail=17, n=8, w=256)
        step = 1
    flush("group kernel %s" % case)
    inp = synth.make_inputs(wl, DEV)
    got = run_layer(wl, inp)
    for b in range(wl.batch):
        rows = _rows(wl, 0, step, b)
        flush("  batch %d: %d rows" % (b, len(rows)))
        compare_layer(wl, inp, got, rows, b)



def test_group_kernel_large_values():
    """Values scaled by 2^16 (exact in bf16, and in the fp32 block sums): the compressed values then
    reach 2^18 and more, beyond fp16's range, so the value tiles carry power-of-two scales that differ
    from tile to tile.  The branch output must be 2^16 times the unscaled one: the GPU's o_cmp over
    2^16 is held to the oracle's o_cmp of the unscaled values with the usual tolerance (the chosen
    blocks do not depend on V)."""
    import oracle
    from gpu_util import TOL, host, maxabs

    wl = _wl(T=6000, Hq=28, Hkv=4, lead=64, tail=20, n=16, w=512)
    flush("group kernel large values")
    inp = synth.make_inputs(wl, DEV)
    S = 65536.0
    big = dict(inp, v=inp["v"] * S)
    w_v = host(inp["w_v"])
    # the premise: the scaled compressed values need tile scales, and not all the same one
    vc = oracle.compress(host(big["v"][0]), w_v, wl.cmp_block, wl.cmp_stride)
    tmax = [np.abs(vc[i:i + 64, h]).max() for h in range(vc.shape[1]) for i in range(0, vc.shape[0], 64)]
    scales = {max(0, int(np.frexp(m)[1]) - 14) for m in tmax}
    assert len(scales) >= 2 and min(scales) >= 1, scales
    got = run_layer(wl, big)
    ref = run_layer(wl, inp)
    rows = _rows(wl, 0, 7, 0)
    vid = host(inp["is_video"][0])[rows].astype(bool)
    res = oracle.layer(host(inp["q"][0]), host(inp["k"][0]), host(inp["v"][0]), host(inp["w_k"]), w_v,
                       host(inp["gates"][0]), host(inp["is_video"][0]), wl.params(), rows=rows)
    scaled = host(got["o_cmp"][0])[rows][vid] / S
    e = maxabs(scaled, res["o_cmp"][vid])
    flush("  o_cmp / 2^16 vs oracle: %.3g (tile scales %s)" % (e, sorted(scales)))
    assert e <= TOL[wl.dtype]
    # block choice does not depend on the values
    assert np.array_equal(host(got["idx"][0]), host(ref["idx"][0]))


def test_group_kernel_scale_invariance():
    """Queries times 2^12 and keys times 2^-12 (both exact in bf16 and in the fp32 block sums) leave
    every score, hence every output, unchanged: the layer must give bitwise the same outputs and
    blocks as on the unscaled inputs.  The group kernel's fp16 queries and key tiles take range
    scales that move by 12 and -12, and their mantissas, hence the scores, stay the same."""
    from gpu_util import host

    wl = _wl(T=3000, Hq=28, Hkv=4, lead=64, tail=20, n=16, w=512)
    flush("group kernel scale invariance")
    inp = synth.make_inputs(wl, DEV)
    ref = run_layer(wl, inp)
    got = run_layer(wl, dict(inp, q=inp["q"] * 4096.0, k=inp["k"] * (1.0 / 4096.0)))
    for name in ("idx", "o_cmp", "o_slc", "o_swa", "out"):
        assert np.array_equal(host(got[name]), host(ref[name])), name
