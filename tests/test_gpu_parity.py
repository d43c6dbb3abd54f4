"""GPU parity: every entry point of libnsa.so against the fp64 oracle on seeded
inputs, element by element, through the C ABI.

Tolerances: max-abs 1e-4 (fp32 inputs) and 2e-2 (bf16 inputs) on branch and
final outputs; chosen blocks identical wherever the oracle's selection gap
exceeds 1e-3, and a valid selection everywhere else.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import GAP, TOL, check_indices, flush, host, maxabs
from sparse_attention_long_fwd_amd import nsa, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(params=["default", "generic"])
def path(request):
    prev = nsa.set_force_generic(request.param == "generic")
    yield request.param
    nsa.set_force_generic(prev)


def _rand(seed, shape, dtype, scale=1.0):
    return synth.normal(seed, shape, DEV, scale=scale).to(dtype)


def _wl(dtype="bf16", T=1024, Hq=28, Hkv=4, D=128, n=16, w=512, lead=0, tail=0, corr=True, B=1, q_start=0,
        q_len=None, **kw):
    return synth.Workload(name="test", index=9, dtype=dtype, batch=B, kv_len=T,
                          q_len=T - q_start if q_len is None else q_len, q_start=q_start, num_q_heads=Hq,
                          num_kv_heads=Hkv, head_dim=D, top_n=n, window=w, text_lead=lead, text_tail=tail,
                          frame_corr=corr, **kw)


# --------------------------------------------------------------------------- compression
@pytest.mark.parametrize("dtype,B,T,H,D", [("f32", 1, 1024, 1, 64), ("bf16", 2, 1000, 4, 128),
                                           ("bf16", 1, 36352, 4, 128), ("f32", 1, 47, 2, 8), ("bf16", 1, 31, 1, 16)])
def test_compress_kv(dtype, B, T, H, D):
    flush("compress %s B=%d T=%d H=%d D=%d" % (dtype, B, T, H, D))
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    k, v = _rand(101, (B, T, H, D), dt), _rand(102, (B, T, H, D), dt)
    wk = _rand(103, (32,), torch.float32, 1 / math.sqrt(32))
    wv = _rand(104, (32,), torch.float32, 1 / math.sqrt(32))
    kc, vc = nsa.nsa_compress_kv(k, v, wk, wv, 32, 16)
    torch.cuda.synchronize()
    assert kc.shape[1] == nsa.num_cmp_blocks(T, 32, 16)
    for b in range(B):
        rk = oracle.compress(host(k[b]), host(wk), 32, 16)
        rv = oracle.compress(host(v[b]), host(wv), 32, 16)
        for got, ref in ((kc[b], rk), (vc[b], rv)):
            g = host(got).astype(np.float64)
            bound = (2.0 ** -8 * np.abs(ref) + 1e-5) if dtype == "bf16" else 1e-5
            assert np.all(np.abs(g - ref) <= bound)


# --------------------------------------------------------------------------- compression branch
@pytest.mark.parametrize("dtype,T,Hq,Hkv,D,lead,tail,q_start", [
    ("f32", 1024, 4, 1, 64, 0, 0, 0),
    ("bf16", 1000, 14, 2, 128, 64, 40, 0),
    ("bf16", 3000, 28, 4, 128, 128, 128, 0),
    ("bf16", 5000, 28, 4, 128, 0, 0, 4900),
])
def test_cmp_attn_scores(dtype, T, Hq, Hkv, D, lead, tail, q_start, path):
    flush("cmp %s T=%d Hq=%d path=%s" % (dtype, T, Hq, path))
    wl = _wl(dtype, T, Hq, Hkv, D, lead=lead, tail=tail, q_start=q_start)
    dt = wl.torch_dtype
    Nc = nsa.num_cmp_blocks(T, 32, 16)
    q = _rand(111, (1, wl.q_len, Hq, D), dt)
    kc = _rand(112, (1, Nc, Hkv, D), dt)
    vc = _rand(113, (1, Nc, Hkv, D), dt)
    vid = synth.video_mask(wl, DEV)
    sh = nsa.make_shape(1, wl.q_len, T, q_start, Hq, Hkv, D)
    pr = nsa.make_params(top_n=16, window=512)
    o, lse, imp = nsa.nsa_cmp_attn_scores(q, kc, vc, sh, pr, is_video=vid)
    torch.cuda.synchronize()
    pos = np.arange(q_start, q_start + wl.q_len)
    ro, rl, ri = oracle.cmp_rows(host(q[0]), pos, host(kc[0]), host(vc[0]), Hq, 32, 16, 64, T, 1 / math.sqrt(D))
    V = host(vid[0]).astype(bool)
    assert maxabs(host(o[0])[V], ro[V]) <= TOL[dtype]
    fin = np.isfinite(rl[V])
    gl = host(lse[0])[V]
    assert np.all(np.isneginf(gl[~fin]))
    assert maxabs(gl[fin], rl[V][fin]) <= 1e-3
    assert maxabs(host(imp[0])[V], ri[V]) <= 2e-4


@pytest.mark.parametrize("want", [("o_cmp",), ("importance",), ("o_cmp", "lse")])
def test_cmp_attn_scores_optional_outputs(want, path):
    """Outputs left NULL are not written; the given ones equal those of a full call."""
    T, Hq, Hkv, D = 2100, 14, 2, 128
    wl = _wl("bf16", T, Hq, Hkv, D, lead=64, tail=20)
    Nc = nsa.num_cmp_blocks(T, 32, 16)
    q = _rand(121, (1, T, Hq, D), torch.bfloat16)
    kc = _rand(122, (1, Nc, Hkv, D), torch.bfloat16)
    vc = _rand(123, (1, Nc, Hkv, D), torch.bfloat16)
    vid = synth.video_mask(wl, DEV)
    sh = nsa.make_shape(1, T, T, 0, Hq, Hkv, D)
    pr = nsa.make_params(top_n=16, window=512)
    full = nsa.nsa_cmp_attn_scores(q, kc, vc, sh, pr, is_video=vid)
    part = nsa.nsa_cmp_attn_scores(q, kc, vc, sh, pr, is_video=vid, want=want)
    torch.cuda.synchronize()
    for name, a_, b_ in zip(("o_cmp", "lse", "importance"), full, part):
        if name in want:
            assert torch.equal(a_, b_), name
        else:
            assert b_ is None


# --------------------------------------------------------------------------- top-n
@pytest.mark.parametrize("n,n_init,n_local,Ns,fine", [(4, 1, 2, 16, False), (16, 1, 2, 568, False),
                                                       (16, 1, 2, 2048, False), (8, 2, 3, 300, False),
                                                       (32, 1, 2, 2048, False), (3, 0, 3, 50, False),
                                                       (16, 1, 2, 5000, False), (32, 1, 2, 4096, True),
                                                       (16, 1, 2, 6000, True)])
def test_topk_blocks_exact(n, n_init, n_local, Ns, fine):
    """Against the oracle bit for bit.  Coarse values (many exact ties, decided by the lower index);
    fine values for rows with more candidates than the per-lane registers hold (the streamed
    threshold path; coarse values there take the arg-max rounds)."""
    flush("topk n=%d Ns=%d fine=%s" % (n, Ns, fine))
    ls = 64
    T = Ns * ls
    R, Hkv = 700, 4
    rng = np.random.default_rng(n * 1000 + Ns)
    pos = np.sort(rng.integers(0, T, R))
    pos[:3] = [0, 63, 64 * 5 + 1]
    pos[-1] = T - 1
    # coarse values: many exact ties, decided by the lower index on both sides
    imp = (rng.integers(0, 40, (R, Hkv, Ns)) / 64.0).astype(np.float32)
    if fine:
        imp = rng.random((R, Hkv, Ns)).astype(np.float32)
    # rows of q given explicitly: one batch element per row keeps arbitrary positions
    sh = nsa.make_shape(R, 1, T, 0, Hkv, Hkv, 8)
    imp_d = torch.from_numpy(imp).to(DEV).view(R, 1, Hkv, Ns)
    got = []
    for r0 in range(0, R, 100):
        rows = list(range(r0, min(R, r0 + 100)))
        for r in rows:
            sh1 = nsa.make_shape(1, 1, T, int(pos[r]), Hkv, Hkv, 8)
            got.append(nsa.nsa_topk_blocks(imp_d[r:r + 1], sh1, nsa.make_params(top_n=n, n_init=n_init,
                                                                                 n_local=n_local)))
    torch.cuda.synchronize()
    got = np.concatenate([host(x).reshape(1, Hkv, n) for x in got])
    ref, _ = oracle.topk_rows(imp.astype(np.float64), pos, ls, n, n_init, n_local)
    assert np.array_equal(got, ref)


def test_topk_blocks_many_rows():
    T, Hkv, n = 36352, 4, 16
    Ns = nsa.num_sel_blocks(T, 64)
    wl = _wl(T=T, lead=256, tail=256)
    rng = np.random.default_rng(5)
    imp = rng.random((1, T, Hkv, Ns)).astype(np.float32)
    vid = synth.video_mask(wl, DEV)
    sh = nsa.make_shape(1, T, T, 0, 28, Hkv, 128)
    got = nsa.nsa_topk_blocks(torch.from_numpy(imp).to(DEV), sh, nsa.make_params(top_n=n), is_video=vid)
    torch.cuda.synchronize()
    V = host(vid[0]).astype(bool)
    rows = np.nonzero(V)[0][::37]
    ref, _ = oracle.topk_rows(imp[0, rows].astype(np.float64), rows, 64, n, 1, 2)
    assert np.array_equal(host(got[0])[rows], ref)
    assert np.all(host(got[0])[~V] == -1)  # text rows untouched (initialised to -1)


# --------------------------------------------------------------------------- selection / window / text rows
def _random_idx(pos, Hkv, n, ls, seed):
    rng = np.random.default_rng(seed)
    R = len(pos)
    idx = np.full((R, Hkv, n), -1, np.int32)
    for r in range(R):
        jt = int(pos[r]) // ls
        for g in range(Hkv):
            forced = {j for j in range(jt + 1) if j < 1 or j > jt - 2}
            free = [j for j in range(jt + 1) if j not in forced]
            k = min(n - len(forced), len(free))
            pick = rng.choice(free, size=k, replace=False).tolist() if k > 0 else []
            s = sorted(forced | set(pick))
            idx[r, g, :len(s)] = s
    return idx


@pytest.mark.parametrize("dtype,T,Hq,Hkv,D,n,w,lead,tail,B", [
    ("f32", 1024, 4, 1, 64, 4, 128, 0, 0, 1),
    ("bf16", 1100, 14, 2, 128, 16, 512, 64, 76, 1),
    ("bf16", 4096, 28, 4, 128, 16, 512, 256, 256, 1),
    ("bf16", 700, 28, 4, 128, 8, 256, 0, 0, 2),
])
def test_sparse_attn_fwd(dtype, T, Hq, Hkv, D, n, w, lead, tail, B, path):
    flush("sparse %s T=%d n=%d w=%d B=%d path=%s" % (dtype, T, n, w, B, path))
    wl = _wl(dtype, T, Hq, Hkv, D, n=n, w=w, lead=lead, tail=tail, B=B)
    dt = wl.torch_dtype
    inp = synth.make_inputs(wl, DEV)
    q, k, v, g, vid = inp["q"], inp["k"], inp["v"], inp["gates"], inp["is_video"]
    ocmp = _rand(121, tuple(q.shape), dt)
    pos = np.arange(T)
    idx = np.stack([_random_idx(pos, Hkv, n, 64, 7 + b) for b in range(B)])
    idx_d = torch.from_numpy(idx).to(DEV)
    sh = nsa.shape_of(q, k)
    pr = nsa.make_params(top_n=n, window=w)
    out, o_slc, o_swa = torch.zeros_like(q), torch.zeros_like(q), torch.zeros_like(q)
    nsa.nsa_sparse_attn_fwd(q, k, v, sh, pr, idx_d, is_video=vid, o_cmp=ocmp, gates=g, out=out, o_slc=o_slc,
                            o_swa=o_swa)
    torch.cuda.synchronize()
    s = 1 / math.sqrt(D)
    for b in range(B):
        V = host(vid[b]).astype(bool)
        vr = np.nonzero(V)[0]
        tr = np.nonzero(~V)[0]
        qh, kh, vh = host(q[b]), host(k[b]), host(v[b])
        rs, rw = oracle.sparse_rows(qh[vr], vr, kh, vh, idx[b][vr], 64, w, s)
        assert maxabs(host(o_slc[b])[vr], rs) <= TOL[dtype]
        assert maxabs(host(o_swa[b])[vr], rw) <= TOL[dtype]
        gg = host(g[b])[vr].astype(np.float64)
        ref = gg[..., 0:1] * host(ocmp[b])[vr] + gg[..., 1:2] * rs + gg[..., 2:3] * rw
        assert maxabs(host(out[b])[vr], ref) <= TOL[dtype]
        if tr.size:
            rd, _ = oracle.dense_rows(qh[tr], tr, kh, vh, s)
            assert maxabs(host(out[b])[tr], rd) <= TOL[dtype]


def test_sparse_attn_fwd_future_blocks(path):
    """Caller-given sets may list blocks after the row's own block: they hold no key u <= t and
    contribute nothing (the oracle skips them too), on both paths."""
    T, Hq, Hkv, D, n, w = 2000, 14, 2, 128, 8, 256
    wl = _wl("bf16", T, Hq, Hkv, D, n=n, w=w, lead=64, tail=0)
    inp = synth.make_inputs(wl, DEV)
    q, k, v, g, vid = inp["q"], inp["k"], inp["v"], inp["gates"], inp["is_video"]
    ocmp = _rand(131, tuple(q.shape), torch.bfloat16)
    pos = np.arange(T)
    Ns = nsa.num_sel_blocks(T, 64)
    idx = _random_idx(pos, Hkv, n, 64, 17)
    rng = np.random.default_rng(3)
    for r in range(T):
        jt = r // 64
        for gg in range(Hkv):
            s = [int(x) for x in idx[r, gg] if x >= 0]
            free = [x for x in s if 0 < x < jt - 1]
            later = list(range(jt + 1, Ns))
            if free and later and rng.random() < 0.5:
                s.remove(free[0])
                s.append(int(rng.choice(later)))
            s = sorted(s)
            idx[r, gg] = -1
            idx[r, gg, :len(s)] = s
    sh = nsa.shape_of(q, k)
    pr = nsa.make_params(top_n=n, window=w)
    out, o_slc = torch.zeros_like(q), torch.zeros_like(q)
    nsa.nsa_sparse_attn_fwd(q, k, v, sh, pr, torch.from_numpy(idx).to(DEV), is_video=vid, o_cmp=ocmp, gates=g,
                            out=out, o_slc=o_slc)
    torch.cuda.synchronize()
    V = host(vid[0]).astype(bool)
    vr = np.nonzero(V)[0]
    rs, rw = oracle.sparse_rows(host(q[0])[vr], vr, host(k[0]), host(v[0]), idx[vr], 64, w, 1 / math.sqrt(D))
    assert maxabs(host(o_slc[0])[vr], rs) <= TOL["bf16"]
    gg = host(g[0])[vr].astype(np.float64)
    ref = gg[..., 0:1] * host(ocmp[0])[vr] + gg[..., 1:2] * rs + gg[..., 2:3] * rw
    assert maxabs(host(out[0])[vr], ref) <= TOL["bf16"]


# --------------------------------------------------------------------------- whole layer
def run_layer(wl, inp, **kw):
    q = inp["q"]
    B, Tq, Hq, D = q.shape
    Hkv = inp["k"].shape[2]
    sh = nsa.make_shape(B, Tq, wl.kv_len, wl.q_start, Hq, Hkv, D)
    pr = nsa.make_params(**{k: v for k, v in wl.params().items()})
    o_cmp, o_slc, o_swa = torch.zeros_like(q), torch.zeros_like(q), torch.zeros_like(q)
    idx = torch.full((B, Tq, Hkv, wl.top_n), -1, dtype=torch.int32, device=DEV)
    out = nsa.nsa_hybrid_layer_fwd(q, inp["k"], inp["v"], inp["gates"], sh, pr, w_k=inp["w_k"], w_v=inp["w_v"],
                                   is_video=inp["is_video"], o_cmp=o_cmp, o_slc=o_slc, o_swa=o_swa,
                                   block_idx_out=idx, **kw)
    torch.cuda.synchronize()
    return dict(out=out, o_cmp=o_cmp, o_slc=o_slc, o_swa=o_swa, idx=idx)


def compare_layer(wl, inp, got, rows, b=0, kc=None, vc=None):
    """Oracle on the chosen rows of batch element b; assert the parity rules.  inp may hold
    per-branch keys / values (k_s, v_s: selection; k_w, v_w: window and text rows)."""
    dtype = wl.dtype
    q = host(inp["q"][b])
    k, v = host(inp["k"][b]), host(inp["v"][b])
    okw = {}
    if "k_s" in inp:
        okw = dict(kv_slc=(host(inp["k_s"][b]), host(inp["v_s"][b])), kv_swa=(host(inp["k_w"][b]), host(inp["v_w"][b])))
    res = oracle.layer(q, k, v, host(inp["w_k"]), host(inp["w_v"]), host(inp["gates"][b]),
                       host(inp["is_video"][b]), wl.params(), q_start=wl.q_start, rows=rows, kc=kc, vc=vc, **okw)
    V = host(inp["is_video"][b])[rows].astype(bool)
    pos = rows + wl.q_start
    tol = TOL[dtype]
    stats = {}
    if V.any():
        same = check_indices(host(got["idx"][b])[rows][V], res["idx"][V], res["gap"][V], res["imp"][V], pos[V],
                             wl.sel_block, wl.top_n, wl.n_init, wl.n_local)
        rows_same = same.all(axis=1)
        stats["decided"] = float((res["gap"][V] > GAP).mean())
        stats["idx_equal"] = float(same.mean())
        # Rows whose GPU set differs from the oracle's (only where the oracle's own choice is
        # undecided, checked above): the selection and final outputs are compared against the
        # oracle run on the GPU's set, so no row is left out of the output comparison.
        ref_slc = res["o_slc"][V].copy()
        ref_out = res["out"][V].copy()
        sub = np.nonzero(~rows_same)[0]
        stats["substituted_rows"] = int(sub.size)
        if sub.size:
            vrows = rows[V][sub]
            ks, vs = okw["kv_slc"] if okw else (k, v)
            gidx = host(got["idx"][b])[vrows]
            scale = oracle.default_scale(q.shape[-1], wl.params().get("scale", 0.0))
            o_sub, _ = oracle.sparse_rows(q[vrows], vrows + wl.q_start, ks, vs, gidx, wl.sel_block, wl.window,
                                          scale, swa=False)
            gg = host(inp["gates"][b])[vrows].astype(np.float64)
            ref_slc[sub] = o_sub
            ref_out[sub] = (gg[..., 0:1] * res["o_cmp"][V][sub] + gg[..., 1:2] * o_sub +
                            gg[..., 2:3] * res["o_swa"][V][sub])
        e_cmp = maxabs(host(got["o_cmp"][b])[rows][V], res["o_cmp"][V])
        e_swa = maxabs(host(got["o_swa"][b])[rows][V], res["o_swa"][V])
        e_slc = maxabs(host(got["o_slc"][b])[rows][V], ref_slc)
        e_out = maxabs(host(got["out"][b])[rows][V], ref_out)
        stats.update(cmp=e_cmp, swa=e_swa, slc=e_slc, out=e_out)
        ecmp_rows = np.abs(host(got["o_cmp"][b])[rows][V] - res["o_cmp"][V]).max(axis=(1, 2))
        stats["cmp_worst_pos"] = int(pos[V][np.argmax(ecmp_rows)])
        assert e_cmp <= tol and e_swa <= tol and e_slc <= tol and e_out <= tol, stats
    if (~V).any():
        e_txt = maxabs(host(got["out"][b])[rows][~V], res["out"][~V])
        stats["text"] = e_txt
        assert e_txt <= tol, stats
    flush("  parity %s" % stats)
    return stats


@pytest.mark.parametrize("case", ["tiny", "bf16-4k", "bf16-ragged", "bf16-batch2", "bf16-g4", "bf16-g8"])
def test_layer_small(case, path):
    if case == "tiny":
        wl = synth.WORKLOADS["tiny"]
    elif case == "bf16-4k":
        wl = _wl(T=4096, lead=256, tail=256)
    elif case == "bf16-ragged":
        wl = _wl(T=1000 + 37, Hq=14, Hkv=2, lead=64, tail=13, n=6, w=100)
    elif case == "bf16-g4":  # 4 query heads per KV head
        wl = _wl(T=2600, Hq=8, Hkv=2, lead=64, tail=30, n=8, w=256)
    elif case == "bf16-g8":  # 8 query heads per KV head (one importance buffer in LDS)
        wl = _wl(T=5000, Hq=16, Hkv=2, lead=64, tail=30, n=8, w=256)
    else:
        wl = _wl(T=900, B=2, lead=128, tail=0, n=8, w=256)
    flush("layer %s path=%s" % (case, path))
    inp = synth.make_inputs(wl, DEV)
    got = run_layer(wl, inp)
    for b in range(wl.batch):
        compare_layer(wl, inp, got, np.arange(wl.q_len), b)


def _sample_rows(wl, per_frame=1, seed=0, text=8, edge=64):
    """Deterministic row sample: the first and last rows, a few text rows, and
    one row per `stride` video rows at a seeded offset."""
    T = wl.q_len
    rng = np.random.default_rng(seed)
    rows = set(range(min(edge, T))) | set(range(max(0, T - edge), T))
    vid = host(synth.video_mask(wl))[0].astype(bool)
    tr = np.nonzero(~vid)[0]
    if tr.size:
        rows |= set(rng.choice(tr, size=min(text, tr.size), replace=False).tolist())
    stride = max(64, T // 400)
    off = int(rng.integers(0, stride))
    rows |= set(range(off, T, stride))
    return np.array(sorted(r for r in rows if 0 <= r < T), dtype=np.int64)


@pytest.mark.parametrize("name", ["36k", "128k"])
def test_layer_full_size_sampled(name):
    wl = synth.WORKLOADS[name]
    flush("layer full-size %s" % name)
    inp = synth.make_inputs(wl, DEV)
    got = run_layer(wl, inp)
    rows = _sample_rows(wl, seed=wl.index)
    flush("  %d sampled rows" % len(rows))
    compare_layer(wl, inp, got, rows)


@pytest.mark.parametrize("variant", range(len(synth.SWEEP_VARIANTS)))
def test_layer_sweep_sampled(variant):
    n, w, gates = synth.SWEEP_VARIANTS[variant]
    wl = synth.WORKLOADS["sweep"].with_(top_n=n, window=w, gates=gates)
    flush("sweep n=%d w=%d gates=%s" % (n, w, gates))
    inp = synth.make_inputs(wl, DEV)
    got = run_layer(wl, inp)
    rows = _sample_rows(wl, seed=variant, text=4, edge=16)[::3]
    compare_layer(wl, inp, got, rows)


@pytest.mark.parametrize("n,w", [(8, 1024), (23, 64)])
def test_layer_budget_points_sampled(n, w):
    """The ends of the fixed-budget (64 n + w = 1536) performance surface at 128K."""
    wl = synth.WORKLOADS["128k"].with_(top_n=n, window=w)
    flush("budget point n=%d w=%d" % (n, w))
    inp = synth.make_inputs(wl, DEV)
    got = run_layer(wl, inp)
    rows = _sample_rows(wl, seed=n, text=4, edge=16)[::3]
    compare_layer(wl, inp, got, rows)


def test_decode_with_compressed_cache():
    wl = synth.WORKLOADS["decode"]
    flush("decode B=%d L=%d" % (wl.batch, wl.kv_len))
    inp = synth.make_inputs(wl, DEV)
    # the compressed cache comes from the oracle, rounded to bf16, and feeds both sides
    kcs, vcs = [], []
    for b in range(wl.batch):
        kcs.append(oracle.compress(host(inp["k"][b]), host(inp["w_k"]), 32, 16))
        vcs.append(oracle.compress(host(inp["v"][b]), host(inp["w_v"]), 32, 16))
    kc = torch.from_numpy(np.stack(kcs)).to(DEV).to(torch.bfloat16)
    vc = torch.from_numpy(np.stack(vcs)).to(DEV).to(torch.bfloat16)
    got = run_layer(wl, inp, k_cmp_in=kc, v_cmp_in=vc)
    for b in range(wl.batch):
        compare_layer(wl, inp, got, np.arange(1), b, kc=host(kc[b]).astype(np.float64),
                      vc=host(vc[b]).astype(np.float64))


@pytest.mark.parametrize("case", ["short", "no-cmp-block", "n-covers-all", "window-covers-all", "all-text"])
def test_layer_edge_cases(case, path):
    kw = dict(T=300, Hq=14, Hkv=2, lead=0, tail=0, n=8, w=64)
    if case == "short":
        kw.update(T=70)
    elif case == "no-cmp-block":
        kw.update(T=31)
    elif case == "n-covers-all":
        kw.update(T=500, n=16)
    elif case == "window-covers-all":
        kw.update(T=400, w=4096)
    elif case == "all-text":
        kw.update(lead=300)
    wl = _wl(**kw)
    flush("edge %s path=%s" % (case, path))
    inp = synth.make_inputs(wl, DEV)
    got = run_layer(wl, inp)
    compare_layer(wl, inp, got, np.arange(wl.q_len))


@pytest.mark.parametrize("n,n_init,n_local", [(32, 0, 1), (3, 1, 2), (12, 3, 4), (5, 0, 5), (6, 2, 1)])
def test_layer_selection_params(n, n_init, n_local, path):
    """Top-n inside the layer for other forced-block counts: no leading block, no free place
    left (n = n_init + n_local), and enough rows past several 1024-token key tiles for the
    candidate lists to be cut down many times."""
    wl = _wl(T=5200, Hq=14, Hkv=2, lead=96, tail=40, n=n, w=256, n_init=n_init, n_local=n_local)
    flush("selection n=%d n_init=%d n_local=%d path=%s" % (n, n_init, n_local, path))
    inp = synth.make_inputs(wl, DEV)
    got = run_layer(wl, inp)
    rows = np.unique(np.concatenate([np.arange(0, 300), np.arange(300, wl.q_len, 7), np.arange(wl.q_len - 64,
                                                                                               wl.q_len)]))
    compare_layer(wl, inp, got, rows)


@pytest.mark.parametrize("q_start", [1024, 1000])
def test_layer_query_block(q_start, path):
    """A block of query rows at the end of the sequence (chunked prefill): rows start at position
    q_start, aligned to 32 (the window pass then takes over the forced local blocks) or not."""
    wl = _wl(T=3000, Hq=14, Hkv=2, lead=40, tail=60, n=8, w=256, q_start=q_start)
    flush("query block q_start=%d path=%s" % (q_start, path))
    inp = synth.make_inputs(wl, DEV)
    got = run_layer(wl, inp)
    compare_layer(wl, inp, got, np.arange(wl.q_len))


def test_layer_deterministic():
    wl = _wl(T=3000, lead=128, tail=128)
    inp = synth.make_inputs(wl, DEV)
    a = run_layer(wl, inp)
    b = run_layer(wl, inp)
    for key in ("out", "o_cmp", "o_slc", "o_swa", "idx"):
        assert torch.equal(a[key], b[key]), key


def test_layer_side_stream_equals_in_order():
    """The window pass forked onto the library's second stream (the default) and the two passes in
    order on the caller's stream (as while phase timing is on) give the same bits, text rows
    included."""
    wl = _wl(T=3000, lead=128, tail=128)
    inp = synth.make_inputs(wl, DEV)
    a = run_layer(wl, inp)
    nsa.profile_enable(True)
    try:
        b = run_layer(wl, inp)
        torch.cuda.synchronize()
    finally:
        nsa.profile_enable(False)
    for key in ("out", "o_cmp", "o_slc", "o_swa", "idx"):
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("case", ["internal-compress", "text-row", "early-row", "batch3-mixed"])
def test_decode_single_row(case, path):
    """One query row per sequence (the split decode kernels), compressed inside the layer."""
    T, B, q_start = 5000, 1, 4999
    lead, tail = 0, 0
    if case == "text-row":
        tail = 1
    elif case == "early-row":
        T, q_start = 4000, 70
    elif case == "batch3-mixed":
        B, T, q_start = 3, 3000, 2500
    wl = _wl(T=T, B=B, q_start=q_start, q_len=1, lead=lead, tail=tail)
    flush("decode %s path=%s" % (case, path))
    inp = synth.make_inputs(wl, DEV)
    if case == "batch3-mixed":
        inp["is_video"][1] = 0  # the middle sequence's row is a text row
    got = run_layer(wl, inp)
    for b in range(B):
        compare_layer(wl, inp, got, np.arange(1), b)


# --------------------------------------------------------------------------- keys / values per branch
def run_layer_branch_kv(wl, inp, **kw):
    q = inp["q"]
    B, Tq, Hq, D = q.shape
    Hkv = inp["k"].shape[2]
    sh = nsa.make_shape(B, Tq, wl.kv_len, wl.q_start, Hq, Hkv, D)
    pr = nsa.make_params(**wl.params())
    o_cmp, o_slc, o_swa = torch.zeros_like(q), torch.zeros_like(q), torch.zeros_like(q)
    idx = torch.full((B, Tq, Hkv, wl.top_n), -1, dtype=torch.int32, device=DEV)
    out = nsa.nsa_hybrid_layer_fwd_branch_kv(q, (inp["k"], inp["v"]), (inp["k_s"], inp["v_s"]),
                                             (inp["k_w"], inp["v_w"]), inp["gates"], sh, pr, w_k=inp["w_k"],
                                             w_v=inp["w_v"], is_video=inp["is_video"], o_cmp=o_cmp, o_slc=o_slc,
                                             o_swa=o_swa, block_idx_out=idx, **kw)
    torch.cuda.synchronize()
    return dict(out=out, o_cmp=o_cmp, o_slc=o_slc, o_swa=o_swa, idx=idx)


def _branch_inputs(wl):
    inp = synth.make_inputs(wl, DEV)
    for tag, off in (("s", 40), ("w", 80)):
        other = synth.make_inputs(wl, DEV, batch_offset=off)
        inp["k_" + tag], inp["v_" + tag] = other["k"], other["v"]
    return inp


@pytest.mark.parametrize("case", ["bf16-4k", "bf16-ragged-batch2"])
def test_layer_branch_kv(case, path):
    if case == "bf16-4k":
        wl = _wl(T=4096, lead=256, tail=256)
    else:
        wl = _wl(T=1000 + 37, B=2, Hq=14, Hkv=2, lead=64, tail=13, n=6, w=100)
    flush("branch kv %s path=%s" % (case, path))
    inp = _branch_inputs(wl)
    got = run_layer_branch_kv(wl, inp)
    for b in range(wl.batch):
        compare_layer(wl, inp, got, np.arange(wl.q_len), b)


def test_layer_branch_kv_full_size_sampled():
    wl = synth.WORKLOADS["36k"]
    flush("branch kv 36k")
    inp = _branch_inputs(wl)
    got = run_layer_branch_kv(wl, inp)
    compare_layer(wl, inp, got, _sample_rows(wl, seed=7, text=8, edge=32)[::2])


def test_layer_branch_kv_shared_equals_layer():
    wl = _wl(T=3000, lead=128, tail=128)
    inp = synth.make_inputs(wl, DEV)
    inp["k_s"], inp["v_s"], inp["k_w"], inp["v_w"] = inp["k"], inp["v"], inp["k"], inp["v"]
    a = run_layer(wl, inp)
    b = run_layer_branch_kv(wl, inp)
    for key in ("out", "o_cmp", "o_slc", "o_swa", "idx"):
        assert torch.equal(a[key], b[key]), key
