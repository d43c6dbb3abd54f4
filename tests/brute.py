"""Dense-mask NumPy brute force of the hybrid layer, for tiny shapes.

It takes a different route from the oracle on purpose: every branch is written
as a full T x T (or T x Nc) masked softmax, compression is a membership matrix
product, block importance goes through an explicit overlap matrix built from
token membership, and top-n uses Python's stable sort.  Agreement between the
two is one of the pins of the oracle.
"""
from __future__ import annotations

import math

import numpy as np


def cmp_membership(T, l, d):
    """A[i, u] = 1 when token u lies in compressed block i."""
    Nc = (T - l) // d + 1 if T >= l else 0
    A = np.zeros((Nc, T))
    for i in range(Nc):
        A[i, i * d:i * d + l] = 1.0
    return A


def compress(x, w, l, d):
    T = x.shape[0]
    Nc = (T - l) // d + 1 if T >= l else 0
    W = np.zeros((Nc, T))
    for i in range(Nc):
        W[i, i * d:i * d + l] = np.asarray(w, dtype=np.float64)
    return np.einsum("it,thd->ihd", W, np.asarray(x, dtype=np.float64))


def overlap_matrix(T, l, d, ls):
    """Omega[i, j] = (tokens of compressed block i inside selection block j) / l."""
    A = cmp_membership(T, l, d)
    Ns = (T + ls - 1) // ls
    S = np.zeros((T, Ns))
    S[np.arange(T), np.arange(T) // ls] = 1.0
    return A @ S / l


def masked_attention(q, kk, vv, mask, scale):
    """q [Tq, D], kk/vv [Tk, D], mask [Tq, Tk] bool -> out [Tq, D], p [Tq, Tk]."""
    z = scale * (q @ kk.T)
    z = np.where(mask, z, -np.inf)
    m = np.max(z, axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(mask, np.exp(z - m), 0.0)
    s = e.sum(axis=1, keepdims=True)
    p = np.where(s > 0, e / np.where(s > 0, s, 1.0), 0.0)
    return p @ vv, p


def topk(imp_row, t, ls, n, n_init, n_local):
    jt = t // ls
    J = list(range(jt + 1))
    F = [j for j in J if j < n_init or j > jt - n_local]
    free = sorted((j for j in J if j not in F), key=lambda j: (-imp_row[j], j))
    k = max(0, n - len(F))
    S = sorted(F + free[:k])
    return S + [-1] * (n - len(S))


def layer(q, k, v, w_k, w_v, gates, is_video, params, q_start=0):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, Hq, D = q.shape
    T, Hkv, _ = k.shape
    G = Hq // Hkv
    l, d, ls = params["cmp_block"], params["cmp_stride"], params["sel_block"]
    n, n_init, n_local, w = params["top_n"], params["n_init"], params["n_local"], params["window"]
    scale = params.get("scale", 0.0) or 1.0 / math.sqrt(D)
    kc, vc = compress(k, w_k, l, d), compress(v, w_v, l, d)
    Nc = kc.shape[0]
    Ns = (T + ls - 1) // ls
    Om = overlap_matrix(T, l, d, ls)
    pos = np.arange(Tq) + q_start
    u = np.arange(T)
    causal = u[None, :] <= pos[:, None]
    cmask = (np.arange(Nc)[None, :] * d + l - 1) <= pos[:, None]
    band = causal & (u[None, :] > pos[:, None] - w)
    res = {x: np.zeros((Tq, Hq, D)) for x in ("o_cmp", "o_slc", "o_swa", "dense", "out")}
    res["imp"] = np.zeros((Tq, Hkv, Ns))
    res["idx"] = np.full((Tq, Hkv, n), -1, dtype=np.int64)
    for h in range(Hq):
        g = h // G
        res["o_cmp"][:, h], p = masked_attention(q[:, h], kc[:, g], vc[:, g], cmask, scale)
        res["imp"][:, g] += p @ Om
        res["o_swa"][:, h], _ = masked_attention(q[:, h], k[:, g], v[:, g], band, scale)
        res["dense"][:, h], _ = masked_attention(q[:, h], k[:, g], v[:, g], causal, scale)
    for r in range(Tq):
        for g in range(Hkv):
            res["idx"][r, g] = topk(res["imp"][r, g], pos[r], ls, n, n_init, n_local)
    for h in range(Hq):
        g = h // G
        sel = np.zeros((Tq, Ns), dtype=bool)
        for r in range(Tq):
            for j in res["idx"][r, g]:
                if j >= 0:
                    sel[r, j] = True
        smask = causal & sel[:, u // ls]
        res["o_slc"][:, h], _ = masked_attention(q[:, h], k[:, g], v[:, g], smask, scale)
    gg = np.asarray(gates, dtype=np.float64)
    nsa = gg[..., 0:1] * res["o_cmp"] + gg[..., 1:2] * res["o_slc"] + gg[..., 2:3] * res["o_swa"]
    vid = np.asarray(is_video).astype(bool)
    res["out"] = np.where(vid[:, None, None], nsa, res["dense"])
    return res
