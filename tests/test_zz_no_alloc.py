"""nsa_decode_fwd_noalloc (the decode step with the library's own device scratch, for callers that
cannot allocate) against nsa_decode_fwd with a caller workspace, through the C ABI: two calls in a
row, the second on a smaller batch, so the second runs over scratch the first left behind.  The
kernels are the same, so every output must be identical bit for bit."""
import numpy as np
import pytest
import torch

from gpu_util import flush
from sparse_attention_long_fwd_amd import nsa, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _batch(lens, cap, paged, text, seed_index):
    wl = synth.WORKLOADS["decode_varlen"].with_(batch=len(lens), kv_len=cap, q_start=cap - 1, index=seed_index)
    inp = synth.make_inputs(wl, DEV)
    for b in text:
        inp["is_video"][b] = 0
    B, T, Hkv, D = inp["k"].shape
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    k, v, table = inp["k"], inp["v"], None
    if paged:
        mp = T // nsa.PAGE_ROWS
        perm = torch.from_numpy(np.random.default_rng(seed_index).permutation(B * mp)).to(DEV)
        table = perm.view(B, mp).to(torch.int32)
        k = torch.empty(B * mp, nsa.PAGE_ROWS, Hkv, D, dtype=inp["k"].dtype, device=DEV)
        v = torch.empty_like(k)
        k[perm] = inp["k"].view(B * mp, nsa.PAGE_ROWS, Hkv, D)
        v[perm] = inp["v"].view(B * mp, nsa.PAGE_ROWS, Hkv, D)
    nc = nsa.num_cmp_blocks(T, 32, 16)
    kc = torch.zeros(B, nc, Hkv, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    nsa.nsa_compress_append(k, v, inp["w_k"], inp["w_v"], kc, vc, T, T, kv_lens=lens_t, page_table=table)
    return wl, inp, dict(k=k, v=v, kc=kc, vc=vc, lens=lens_t, table=table)


def _run(fn, wl, inp, c, **kw):
    q = inp["q"]
    B, _, Hq, D = q.shape
    sh = nsa.make_shape(B, 1, wl.kv_len, 0, Hq, c["k"].shape[-2], D)
    pr = nsa.make_params(**wl.params())
    # the branch outputs of text rows are left untouched by both calls: start from zeros
    got = dict(out=torch.empty_like(q), o_cmp=torch.zeros_like(q), o_slc=torch.zeros_like(q),
               o_swa=torch.zeros_like(q),
               idx=torch.full((B, 1, c["k"].shape[-2], wl.top_n), -7, dtype=torch.int32, device=DEV))
    fn(q, c["k"], c["v"], c["kc"], c["vc"], inp["gates"], sh, pr, kv_lens=c["lens"], page_table=c["table"],
       is_video=inp["is_video"], out=got["out"], o_cmp=got["o_cmp"], o_slc=got["o_slc"], o_swa=got["o_swa"],
       block_idx_out=got["idx"], **kw)
    return got


def test_decode_noalloc_matches_workspace_call():
    cases = [
        # 16 sequences of 4K..64K tokens in a paged cache (the variable-length decode workload)
        ("16 x (4K..64K) paged", synth.decode_lengths(synth.WORKLOADS["decode_varlen"]), 65536, True, (5,), 6),
        # then a smaller batch over the scratch the first call left: 3 short sequences, contiguous
        ("3 x (20..5000) contiguous", [5000, 20, 1013], 5120, False, (1,), 12),
    ]
    for name, lens, cap, paged, text, seed in cases:
        flush("noalloc decode %s" % name)
        wl, inp, c = _batch(lens, cap, paged, text, seed)
        ws_size = nsa.nsa_decode_workspace_size(nsa.make_shape(len(lens), 1, cap, 0, 28, 4, 128),
                                                nsa.make_params(**wl.params()), nsa.NSA_BF16)
        ref = _run(nsa.nsa_decode_fwd, wl, inp, c,
                   workspace=torch.empty(ws_size, dtype=torch.uint8, device=DEV))
        torch.cuda.synchronize()
        got = _run(nsa.nsa_decode_fwd_noalloc, wl, inp, c)
        torch.cuda.synchronize()
        for key in ("out", "o_cmp", "o_slc", "o_swa", "idx"):
            assert torch.equal(got[key], ref[key]), (name, key)
        vid = inp["is_video"][:, 0].bool()
        assert (got["idx"][vid] != -7).all()  # every video row's block ids written
        # twice more in a row on the same inputs: the scratch's old contents change nothing
        again = _run(nsa.nsa_decode_fwd_noalloc, wl, inp, c)
        torch.cuda.synchronize()
        for key in ("out", "idx"):
            assert torch.equal(again[key], ref[key]), (name, key, "repeat")
        del inp, c
