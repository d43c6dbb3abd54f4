"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties one oracle function to something other than itself: a closed
form, a special case that reduces to a textbook routine (torch's scaled
dot-product attention in float64), a dense-mask brute force written along a
different route (tests/brute.py), an invariant, or the pages' own numbers.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import brute
import oracle
from sparse_attention_long_fwd_amd import accounting, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
P = dict(cmp_block=32, cmp_stride=16, sel_block=64, top_n=4, n_init=1, n_local=2, window=128, scale=0.0)


def rnd(seed, *shape):
    return synth.normal(seed, shape).numpy().astype(np.float32)


def small_params(**kw):
    p = dict(cmp_block=8, cmp_stride=4, sel_block=16, top_n=4, n_init=1, n_local=2, window=24, scale=0.0)
    p.update(kw)
    return p


# --------------------------------------------------------------------------- generator
def test_splitmix64_matches_definition():
    # The first output of SplitMix64 seeded with 0, and the plain big-int definition.
    assert synth.splitmix64_reference(0, 1)[0] == 0xE220A8397B1DCDAF
    for seed in (0, 1, 12345, 2**63 + 7):
        ref = synth.splitmix64_reference(seed, 257)
        got = [int(x) & (2**64 - 1) for x in synth.splitmix64_words(seed, 0, 257)]
        assert got == ref
    # counter-based: a window starting mid-stream equals the same slice
    ref = synth.splitmix64_reference(99, 40)
    got = [int(x) & (2**64 - 1) for x in synth.splitmix64_words(99, 30, 10)]
    assert got == ref[30:40]


def test_box_muller_moments_and_chunking():
    x = synth.normal(5, (400000,)).numpy()
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    assert abs(np.mean(x ** 3)) < 0.03 and abs(np.mean(x ** 4) - 3) < 0.05
    # odd offsets inside a chunk give the same numbers as a whole draw
    a = synth.normal(6, (11,)).numpy()
    b = synth.normal(6, (12,)).numpy()
    assert np.array_equal(a, b[:11])


# --------------------------------------------------------------------------- compression
def test_compress_closed_forms():
    T, H, D, l, d = 200, 2, 8, 32, 16
    x = rnd(11, T, H, D)
    Nc = oracle.num_cmp_blocks(T, l, d)
    assert Nc == (T - l) // d + 1 == 11
    for m in (0, 5, 31):
        w = np.zeros(l, np.float32)
        w[m] = 1
        kc = oracle.compress(x, w, l, d)
        assert np.array_equal(kc, x[m: m + d * Nc: d].astype(np.float64))
    kc = oracle.compress(x, np.full(l, 1.0 / l, np.float32), l, d)
    ref = np.stack([x[i * d:i * d + l].astype(np.float64).mean(0) for i in range(Nc)])
    assert np.allclose(kc, ref, atol=1e-6)  # 1/32 is exact in float32
    w1, w2 = rnd(12, l), rnd(13, l)
    lin = oracle.compress(x, w1, l, d) * 2 - oracle.compress(x, w2, l, d) * 3
    ref = oracle.compress(x, (2.0 * w1.astype(np.float64) - 3.0 * w2).astype(np.float32), l, d)
    assert np.allclose(lin, ref, atol=1e-5)
    assert np.allclose(oracle.compress(x, w1, l, d), brute.compress(x, w1, l, d), atol=1e-12)
    assert oracle.num_cmp_blocks(31, 32, 16) == 0 and oracle.compress(x[:31], w1, l, d).shape[0] == 0


# --------------------------------------------------------------------------- compression branch
def test_cmp_against_brute_force_and_closed_forms():
    T, Hq, Hkv, D = 150, 4, 2, 16
    p = small_params()
    l, d, ls = p["cmp_block"], p["cmp_stride"], p["sel_block"]
    q, k, v, w = rnd(21, T, Hq, D), rnd(22, T, Hkv, D), rnd(23, T, Hkv, D), rnd(24, l)
    kc, vc = oracle.compress(k, w, l, d), oracle.compress(v, w, l, d)
    pos = np.arange(T)
    s = 1 / math.sqrt(D)
    o, lse, imp = oracle.cmp_rows(q, pos, kc, vc, Hq, l, d, ls, T, s)
    Nc = kc.shape[0]
    mask = (np.arange(Nc)[None] * d + l - 1) <= pos[:, None]
    Om = brute.overlap_matrix(T, l, d, ls)
    imp_ref = np.zeros_like(imp)
    for h in range(Hq):
        ob, pb = brute.masked_attention(q[:, h].astype(np.float64), kc[:, h // 2], vc[:, h // 2], mask, s)
        assert np.allclose(o[:, h], ob, atol=1e-12)
        imp_ref[:, h // 2] += pb @ Om
    assert np.allclose(imp, imp_ref, atol=1e-12)
    # rows before the first complete block see nothing
    assert np.all(o[: l - 1] == 0) and np.all(np.isneginf(lse[: l - 1])) and np.all(imp[: l - 1] == 0)
    # importance sums to the group size on every row that sees a block
    G = Hq // Hkv
    assert np.allclose(imp[l - 1:].sum(-1), G, atol=1e-12)
    # Q = 0: uniform weights, the mean of the visible compressed values
    o0, lse0, _ = oracle.cmp_rows(np.zeros_like(q), pos, kc, vc, Hq, l, d, ls, T, s)
    for t in (l - 1, 77, T - 1):
        nv = (t + 1 - l) // d + 1
        assert np.allclose(o0[t, 0], vc[:nv, 0].mean(0), atol=1e-12)
        assert abs(lse0[t, 0] - math.log(nv)) < 1e-12
    # constant V = c gives (sum w) * c
    vconst = np.full_like(v, 0.75)
    oc, _, _ = oracle.cmp_rows(q, pos, kc, oracle.compress(vconst, w, l, d), Hq, l, d, ls, T, s)
    assert np.allclose(oc[l - 1:], 0.75 * w.astype(np.float64).sum(), atol=1e-12)


def test_importance_weights_and_identity_case():
    # l = 32, d = 16, ls = 64: block i = 4j-1 .. 4j+3 contributes 1/2, 1, 1, 1, 1/2 to block j
    Om = brute.overlap_matrix(64 * 6, 32, 16, 64)
    j = 3
    assert np.allclose(Om[4 * j - 1: 4 * j + 4, j], [0.5, 1, 1, 1, 0.5])
    assert np.allclose(Om.sum(1), 1.0)
    # l = d = ls: compressed blocks are the selection blocks, so imp = sum over heads of p
    T, Hq, Hkv, D, l = 96, 4, 1, 8, 16
    q, k, v = rnd(31, T, Hq, D), rnd(32, T, Hkv, D), rnd(33, T, Hkv, D)
    w = rnd(34, l)
    kc, vc = oracle.compress(k, w, l, l), oracle.compress(v, w, l, l)
    pos = np.arange(T)
    o, lse, imp = oracle.cmp_rows(q, pos, kc, vc, Hq, l, l, l, T, 0.3)
    Nc = kc.shape[0]
    psum = np.zeros((T, Nc))
    for h in range(Hq):
        z = 0.3 * q[:, h].astype(np.float64) @ kc[:, 0].T
        vis = (np.arange(Nc)[None] * l + l - 1) <= pos[:, None]
        psum += np.where(vis, np.exp(z - lse[:, h:h + 1]), 0.0)
    assert np.allclose(imp[:, 0, :Nc], psum, atol=1e-12)


# --------------------------------------------------------------------------- top-n
def test_topk_worked_example_with_ties():
    ls, n = 64, 6
    t = 64 * 12 + 5          # block of t is 12; forced {0, 11, 12}; 3 free places
    imp = np.zeros((1, 1, 16))
    imp[0, 0, [1, 2, 3, 4, 5, 6, 7, 13]] = [0.5, 0.9, 0.9, 0.1, 0.9, 0.3, 0.9, 5.0]
    idx, gap = oracle.topk_rows(imp, np.array([t]), ls, n, 1, 2)
    # 0.9 is shared by 2, 3, 5, 7: the lower indices win; block 13 lies beyond t
    assert idx[0, 0].tolist() == [0, 2, 3, 5, 11, 12]
    assert gap[0, 0] == 0.0
    # every candidate fits: all blocks up to t, padded
    idx, gap = oracle.topk_rows(imp, np.array([64 * 3 + 1]), ls, n, 1, 2)
    assert idx[0, 0].tolist() == [0, 1, 2, 3, -1, -1] and np.isinf(gap[0, 0])


def test_topk_against_stable_sort():
    rng = np.random.default_rng(0)
    Ns, ls = 40, 16
    imp = np.round(rng.random((300, 2, Ns)), 1)  # coarse values: many planted ties
    pos = rng.integers(0, Ns * ls, 300)
    for n, n_init, n_local in ((4, 1, 2), (8, 2, 1), (16, 1, 2), (40, 1, 2)):
        idx, gap = oracle.topk_rows(imp, pos, ls, n, n_init, n_local)
        for r in range(300):
            for g in range(2):
                ref = brute.topk(imp[r, g], pos[r], ls, n, n_init, n_local)
                assert idx[r, g].tolist() == ref
                jt = pos[r] // ls
                forced = {j for j in range(jt + 1) if j < n_init or j > jt - n_local}
                assert forced <= set(idx[r, g].tolist())
                if n >= jt + 1:
                    assert sorted(x for x in idx[r, g] if x >= 0) == list(range(jt + 1))


# --------------------------------------------------------------------------- selection / window / dense
def _sdpa(q, k, v, mask, s):
    qt = torch.from_numpy(q.astype(np.float64))[None]
    kt = torch.from_numpy(k.astype(np.float64))[None]
    vt = torch.from_numpy(v.astype(np.float64))[None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask),
                                                            scale=s)[0].numpy()


def test_dense_is_textbook_causal_attention():
    T, Hq, Hkv, D = 90, 6, 2, 16
    q, k, v = rnd(41, T, Hq, D), rnd(42, T, Hkv, D), rnd(43, T, Hkv, D)
    s = 1 / math.sqrt(D)
    o, lse = oracle.dense_rows(q, np.arange(T), k, v, s)
    causal = np.tril(np.ones((T, T), dtype=bool))
    for h in range(Hq):
        ref = _sdpa(q[:, h], k[:, h // 3], v[:, h // 3], causal, s)
        assert np.allclose(o[:, h], ref, atol=1e-12)
    z = s * q[5, 0].astype(np.float64) @ k[:6, 0].T.astype(np.float64)
    assert abs(lse[5, 0] - np.log(np.exp(z).sum())) < 1e-12


def test_slc_and_swa_reduce_to_dense_and_brute_force():
    T, Hq, Hkv, D, ls = 130, 4, 1, 8, 16
    q, k, v = rnd(51, T, Hq, D), rnd(52, T, Hkv, D), rnd(53, T, Hkv, D)
    pos = np.arange(T)
    s = 0.4
    dense, _ = oracle.dense_rows(q, pos, k, v, s)
    Ns = (T + ls - 1) // ls
    # every block chosen and a window spanning the sequence: both equal dense causal attention
    allidx = np.tile(np.arange(Ns, dtype=np.int32), (T, Hkv, 1))
    o_slc, o_swa = oracle.sparse_rows(q, pos, k, v, allidx, ls, T, s)
    assert np.allclose(o_slc, dense, atol=1e-12) and np.allclose(o_swa, dense, atol=1e-12)
    # window 1: the row's own value
    _, o1 = oracle.sparse_rows(q, pos, k, v, allidx, ls, 1, s, slc=False)
    assert np.allclose(o1, np.repeat(v[:, :1].astype(np.float64), Hq, 1), atol=1e-15)
    # random valid selections against a dense block mask
    rng = np.random.default_rng(3)
    idx = np.full((T, Hkv, 5), -1, dtype=np.int32)
    for t in range(T):
        jt = t // ls
        cand = sorted(set([0, jt, max(jt - 1, 0)]) | set(rng.integers(0, jt + 1, 2).tolist()))
        idx[t, 0, :len(cand)] = cand
    o_slc, o_swa = oracle.sparse_rows(q, pos, k, v, idx, ls, 20, s)
    u = np.arange(T)
    sel = np.zeros((T, Ns), bool)
    for t in range(T):
        sel[t, idx[t, 0][idx[t, 0] >= 0]] = True
    causal = u[None] <= pos[:, None]
    for h in range(Hq):
        ref, _ = brute.masked_attention(q[:, h].astype(np.float64), k[:, 0].astype(np.float64),
                                        v[:, 0].astype(np.float64), causal & sel[:, u // ls], s)
        assert np.allclose(o_slc[:, h], ref, atol=1e-12)
        band = causal & (u[None] > pos[:, None] - 20)
        ref = _sdpa(q[:, h], k[:, 0], v[:, 0], band, s)
        assert np.allclose(o_swa[:, h], ref, atol=1e-12)


# --------------------------------------------------------------------------- whole layer
def _tiny_inputs(seed, T, Hq, Hkv, D, p, lead=0, tail=0):
    q, k, v = rnd(seed, T, Hq, D), rnd(seed + 1, T, Hkv, D), rnd(seed + 2, T, Hkv, D)
    w = rnd(seed + 3, p["cmp_block"]) / np.float32(math.sqrt(p["cmp_block"]))
    g = (1 / (1 + np.exp(-rnd(seed + 4, T, Hq, 3).astype(np.float64)))).astype(np.float32)
    vid = np.zeros(T, np.uint8)
    vid[lead:T - tail] = 1
    return q, k, v, w, g, vid


def test_layer_against_brute_force():
    T, Hq, Hkv, D = 200, 6, 2, 16
    p = small_params(top_n=5, window=30)
    q, k, v, w, g, vid = _tiny_inputs(60, T, Hq, Hkv, D, p, lead=20, tail=12)
    res = oracle.layer(q, k, v, w, w, g, vid, p)
    ref = brute.layer(q, k, v, w, w, g, vid, p)
    V = vid.astype(bool)
    assert np.array_equal(res["idx"][V], ref["idx"][V])
    for key in ("o_cmp", "o_slc", "o_swa", "imp"):
        assert np.allclose(res[key][V], ref[key][V], atol=1e-12), key
    assert np.allclose(res["out"], ref["out"], atol=1e-12)


def test_layer_one_hot_gates_and_constant_values():
    T, Hq, Hkv, D = 160, 4, 2, 8
    p = small_params()
    q, k, v, w, g, vid = _tiny_inputs(70, T, Hq, Hkv, D, p, lead=16, tail=16)
    base = oracle.layer(q, k, v, w, w, g, vid, p)
    V = vid.astype(bool)
    for b, key in enumerate(("o_cmp", "o_slc", "o_swa")):
        gh = np.zeros_like(g)
        gh[..., b] = 1
        r = oracle.layer(q, k, v, w, w, gh, vid, p)
        assert np.allclose(r["out"][V], base[key][V], atol=0)
        assert np.allclose(r["out"][~V], base["out"][~V], atol=0)  # text rows are ungated
    c = 1.25
    r = oracle.layer(q, k, np.full_like(v, c), w, w, g, vid, p)
    t = np.arange(T)
    seen = ((t + 1 - p["cmp_block"]) >= 0).astype(np.float64)[:, None]
    expect = (g[..., 0] * w.astype(np.float64).sum() * seen + g[..., 1] + g[..., 2]) * c
    assert np.allclose(r["out"][V], np.repeat(expect[V][..., None], D, -1), atol=1e-12)
    assert np.allclose(r["out"][~V], c, atol=1e-12)


def test_layer_text_rows_and_all_text():
    T, Hq, Hkv, D = 120, 4, 1, 8
    p = small_params()
    q, k, v, w, g, vid = _tiny_inputs(80, T, Hq, Hkv, D, p, lead=40, tail=30)
    res = oracle.layer(q, k, v, w, w, g, vid, p)
    dense, _ = oracle.dense_rows(q, np.arange(T), k, v, 1 / math.sqrt(D))
    assert np.allclose(res["out"][~vid.astype(bool)], dense[~vid.astype(bool)], atol=0)
    res = oracle.layer(q, k, v, w, w, g, np.zeros(T, np.uint8), p)
    assert np.allclose(res["out"], dense, atol=0)


def test_layer_causality_and_head_permutation():
    T, Hq, Hkv, D = 180, 6, 2, 8
    p = small_params(top_n=6, window=20)
    q, k, v, w, g, vid = _tiny_inputs(90, T, Hq, Hkv, D, p, lead=8, tail=8)
    res = oracle.layer(q, k, v, w, w, g, vid, p)
    t0 = 101
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[t0 + 1:] += 3.0
    v2[t0 + 1:] -= 2.0
    q2[t0 + 1:] *= -1
    res2 = oracle.layer(q2, k2, v2, w, w, g, vid, p)
    assert np.array_equal(res["out"][: t0 + 1], res2["out"][: t0 + 1])
    # permuting the heads inside a GQA group permutes the outputs
    perm = np.array([2, 0, 1, 5, 3, 4])
    res3 = oracle.layer(q[:, perm], k, v, w, w, g[:, perm], vid, p)
    assert np.allclose(res3["out"], res["out"][:, perm], atol=1e-12)
    assert np.array_equal(res3["idx"], res["idx"])


def test_layer_rows_subset_and_q_start():
    T, Hq, Hkv, D = 150, 4, 2, 8
    p = small_params()
    q, k, v, w, g, vid = _tiny_inputs(95, T, Hq, Hkv, D, p)
    full = oracle.layer(q, k, v, w, w, g, vid, p)
    rows = np.array([3, 40, 99, 149])
    sub = oracle.layer(q, k, v, w, w, g, vid, p, rows=rows)
    assert np.array_equal(sub["out"], full["out"][rows])
    # decode form: one query row at the last position, precomputed compressed cache
    last = oracle.layer(q[-1:], k, v, w, w, g[-1:], vid[-1:], p, q_start=T - 1,
                        kc=full["kc"], vc=full["vc"])
    assert np.allclose(last["out"][0], full["out"][-1], atol=0)


# --------------------------------------------------------------------------- counting
def test_pair_counts_against_key_lists_and_page_identity():
    with open(os.path.join(GOLDEN, "page2_attention_counts.json")) as f:
        page = json.load(f)
    dense = accounting.dense_causal_pairs(page["tokens"])
    assert float("%.2g" % dense) == page["dense_attention_computations"]
    # the pages' own figures are consistent with each other
    assert abs(100 * (1 - page["videonsa_attention_computations"] / page["dense_attention_computations"])
               - page["saving_percent"]) < 0.1
    # closed-form counts equal the number of mask entries the brute force attends
    wl = synth.Workload(name="t", index=0, dtype="f32", batch=1, kv_len=300, q_len=300, q_start=0,
                        num_q_heads=2, num_kv_heads=1, head_dim=8, top_n=3, window=40, text_lead=32,
                        text_tail=20, cmp_block=8, cmp_stride=4, sel_block=16)
    c = accounting.pair_counts(wl)
    T = 300
    pos = np.arange(T)
    vid = (pos >= 32) & (pos < T - 20)
    u = np.arange(T)
    causal = u[None] <= pos[:, None]
    Nc = (T - 8) // 4 + 1
    cmask = (np.arange(Nc)[None] * 4 + 7) <= pos[:, None]
    assert c["cmp"] == 2 * cmask[vid].sum()
    assert c["swa"] == 2 * (causal & (u[None] > pos[:, None] - 40))[vid].sum()
    assert c["text"] == 2 * causal[~vid].sum()
    imp = np.random.default_rng(1).random((T, 1, (T + 15) // 16))
    idx, _ = oracle.topk_rows(imp, pos, 16, 3, 1, 2)
    nslc = 0
    for t in pos[vid]:
        sel = set(idx[t, 0][idx[t, 0] >= 0].tolist())
        nslc += sum(1 for x in range(t + 1) if x // 16 in sel)
    assert c["slc"] == 2 * nslc


def _logit(g):
    return np.log(g) - np.log1p(-g)


def test_gate_proj_closed_forms():
    """Gate projection: x = 0 gives the logistic of the bias at exactly known points; a permutation
    (one-hot) weight reads one hidden channel per gate; a rank-1 weight gives u_f (x . v); the
    logistic is odd about 1/2; the logit is linear in x."""
    rng = np.random.default_rng(7)
    R, K, N = 5, 67, 12
    b = np.array([0.0, math.log(3), -math.log(3), math.log(9)] * 3, dtype=np.float32)
    g0 = oracle.gate_proj(np.zeros((R, K), np.float32), rng.standard_normal((N, K)).astype(np.float32), b)
    want = np.array([0.5, 0.75, 0.25, 0.9] * 3)
    assert np.allclose(g0, want[None, :], atol=1e-6, rtol=0)   # b rounded to float: ~1e-8
    x = rng.standard_normal((R, K)).astype(np.float32)
    perm = rng.permutation(K)[:N]
    w1 = np.zeros((N, K), np.float32)
    w1[np.arange(N), perm] = 1.0
    bb = rng.standard_normal(N).astype(np.float32)
    g1 = oracle.gate_proj(x, w1, bb)
    assert np.allclose(_logit(g1), x[:, perm].astype(np.float64) + bb, atol=1e-9)
    assert g1.shape == (R, N)
    u = rng.standard_normal(N).astype(np.float32)
    v = rng.standard_normal(K).astype(np.float32)
    w2 = (u[:, None].astype(np.float64) * v[None, :]).astype(np.float32)
    g2 = oracle.gate_proj(x, w2)
    xv = x.astype(np.float64) @ v.astype(np.float64)
    assert np.allclose(_logit(g2), xv[:, None] * u[None, :], atol=1e-4)   # w2 rounded to float
    w = (rng.standard_normal((N, K)) / math.sqrt(K)).astype(np.float32)
    gp, gm = oracle.gate_proj(x, w), oracle.gate_proj(-x, w)
    assert np.allclose(gp + gm, 1.0, atol=1e-12)
    # multiples of 2^-10 below 8 in magnitude: their float sums are exact
    xa = (np.round(rng.standard_normal((R, K)) * 1024) / 1024).astype(np.float32)
    xb = (np.round(rng.standard_normal((R, K)) * 1024) / 1024).astype(np.float32)
    s = xa + xb
    assert np.array_equal(s.astype(np.float64), xa.astype(np.float64) + xb)
    lin = _logit(oracle.gate_proj(s, w, bb)) - _logit(oracle.gate_proj(xa, w, bb)) - _logit(
        oracle.gate_proj(xb, w, bb)) + bb
    assert np.allclose(lin, 0.0, atol=1e-9)
    assert np.all((g1 > 0) & (g1 < 1))


def test_layer_branch_kv_independence_and_reductions():
    """Per-branch keys / values: each branch output depends on its own K/V only; with every
    block chosen and a window spanning the sequence, the selection and window outputs are dense
    causal attention over their own K/V (the independent dense path); text rows read the window's
    K/V; all three equal gives the shared-K/V layer."""
    T, Hq, Hkv, D = 200, 4, 2, 16
    q = rnd(61, T, Hq, D)
    k, v = rnd(62, T, Hkv, D), rnd(63, T, Hkv, D)
    k2, v2 = rnd(64, T, Hkv, D), rnd(65, T, Hkv, D)
    k3, v3 = rnd(66, T, Hkv, D), rnd(67, T, Hkv, D)
    w = (rnd(68, 8) / 3).astype(np.float32)
    g = (1 / (1 + np.exp(-rnd(69, T, Hq, 3)))).astype(np.float32)
    vid = np.ones(T, np.uint8)
    vid[:20] = 0
    p = small_params()
    base = oracle.layer(q, k, v, w, w, g, vid, p)
    same = oracle.layer(q, k, v, w, w, g, vid, p, kv_slc=(k, v), kv_swa=(k, v))
    for key in ("o_cmp", "o_slc", "o_swa", "out", "imp"):
        assert np.array_equal(base[key], same[key]), key
    r = oracle.layer(q, k, v, w, w, g, vid, p, kv_slc=(k2, v2), kv_swa=(k3, v3))
    V = vid.astype(bool)
    assert np.array_equal(r["o_cmp"], base["o_cmp"]) and np.array_equal(r["imp"], base["imp"])
    assert np.array_equal(r["idx"], base["idx"])
    assert not np.allclose(r["o_slc"][V], base["o_slc"][V]) and not np.allclose(r["o_swa"][V], base["o_swa"][V])
    # text rows: dense causal attention over the window branch's K/V
    s = 1 / math.sqrt(D)
    tr = np.nonzero(~V)[0]
    dw, _ = oracle.dense_rows(q[tr], tr, k3, v3, s)
    assert np.allclose(r["out"][tr], dw, atol=1e-12)
    # every block chosen (top-n covers all 13 blocks) and a window over the whole sequence
    pall = small_params(top_n=13, window=4096)
    ra = oracle.layer(q, k, v, w, w, g, vid, pall, kv_slc=(k2, v2), kv_swa=(k3, v3))
    vr = np.nonzero(V)[0]
    ds, _ = oracle.dense_rows(q[vr], vr, k2, v2, s)
    dw2, _ = oracle.dense_rows(q[vr], vr, k3, v3, s)
    assert np.allclose(ra["o_slc"][vr], ds, atol=1e-12)
    assert np.allclose(ra["o_swa"][vr], dw2, atol=1e-12)
    gg = g.astype(np.float64)
    assert np.allclose(ra["out"][vr], gg[vr, :, 0:1] * ra["o_cmp"][vr] + gg[vr, :, 1:2] * ds + gg[vr, :, 2:3] * dw2,
                       atol=1e-12)


def _grid(seed, *shape, step=2.0 ** -6, lim=3.0):
    """Seeded values on a 2^-6 grid in [-lim, lim]: x +- 2^-12 stays exact in float32."""
    x = np.clip(np.round(synth.normal(seed, shape).numpy() / step) * step, -lim, lim)
    return x.astype(np.float32)


def test_layer_backward_matches_finite_differences():
    """Backward of sum(dout * out) against central differences of the forward oracle (fp64
    arithmetic on exactly perturbed float inputs, chosen blocks held fixed), over q, k, v, the
    gates and both compression weight vectors, with text and video rows."""
    T, Hq, Hkv, D = 96, 4, 2, 8
    p = small_params(window=20)
    q, k, v = _grid(71, T, Hq, D), _grid(72, T, Hkv, D), _grid(73, T, Hkv, D)
    w_k = (_grid(74, 8) / 4).astype(np.float32)
    w_v = (_grid(75, 8) / 4).astype(np.float32)
    g = (0.25 + 0.5 * (_grid(76, T, Hq, 3) > 0)).astype(np.float32) + _grid(77, T, Hq, 3) / 64
    g = g.astype(np.float32)
    vid = np.ones(T, np.uint8)
    vid[:10] = 0
    vid[-6:] = 0
    dout = _grid(78, T, Hq, D)
    base = oracle.layer(q, k, v, w_k, w_v, g, vid, p)
    idx = base["idx"]
    grad = oracle.layer_bwd(q, k, v, w_k, w_v, g, vid, p, dout, idx=idx)
    eps = 2.0 ** -12
    rng = np.random.default_rng(5)

    def loss(**kw):
        a = dict(q=q, k=k, v=v, w_k=w_k, w_v=w_v, gates=g)
        a.update(kw)
        r = oracle.layer(a["q"], a["k"], a["v"], a["w_k"], a["w_v"], a["gates"], vid, p)
        return float(np.sum(r["out"] * dout)), r["idx"]

    checked = 0
    for name, arr, key in (("q", q, "dq"), ("k", k, "dk"), ("v", v, "dv"), ("gates", g, "dgates"),
                           ("w_k", w_k, "dw_k"), ("w_v", w_v, "dw_v")):
        flat = [tuple(rng.integers(0, s) for s in arr.shape) for _ in range(8)]
        for ix in flat:
            xp, xm = arr.copy(), arr.copy()
            xp[ix] += eps
            xm[ix] -= eps
            lp, ip = loss(**{name: xp})
            lm, im = loss(**{name: xm})
            if not (np.array_equal(ip, idx) and np.array_equal(im, idx)):
                continue  # the perturbation moved a top-n choice: no derivative there
            fd = (lp - lm) / (2 * eps)
            an = grad[key][ix]
            assert abs(fd - an) <= 1e-6 + 1e-5 * abs(an), (name, ix, fd, an)
            checked += 1
    assert checked >= 40
    # text rows have no gate gradient; a zero upstream gradient gives zero gradients
    assert not grad["dgates"][:10].any()
    z = oracle.layer_bwd(q, k, v, w_k, w_v, g, vid, p, np.zeros_like(dout), idx=idx)
    assert all(not z[key].any() for key in ("dq", "dk", "dv", "dgates", "dw_k", "dw_v"))
