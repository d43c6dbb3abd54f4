"""Algorithmic work of the hybrid layer: attended pairs, FLOPs and bytes.

Only pairs the method itself attends are counted; padding, masked tile work and
recomputation are not.  A pair is one (query head, key) product, costing
2*D FLOP for the score and 2*D for the value accumulation.

Per query row at absolute position t (video rows):
  compression  |C(t)| = number of compressed blocks ending at or before t
  selection    tokens u <= t of the chosen blocks; the block holding t is always
               chosen (it is forced), so with |S| = min(n, t // ls + 1) chosen
               blocks this is (|S| - 1) * ls + (t % ls + 1)
  window       min(w, t + 1)
Text rows attend t + 1 keys.
"""
from __future__ import annotations

from typing import Dict

import numpy as np


def cmp_visible(t: np.ndarray, l: int, d: int, T: int) -> np.ndarray:
    t = np.asarray(t, dtype=np.int64)
    nc_total = (T - l) // d + 1 if T >= l else 0
    v = np.where(t + 1 >= l, (t + 1 - l) // d + 1, 0)
    return np.minimum(v, nc_total)


def slc_keys(t: np.ndarray, ls: int, n: int) -> np.ndarray:
    t = np.asarray(t, dtype=np.int64)
    nsel = np.minimum(n, t // ls + 1)
    return (nsel - 1) * ls + (t % ls + 1)


def swa_keys(t: np.ndarray, w: int) -> np.ndarray:
    t = np.asarray(t, dtype=np.int64)
    return np.minimum(w, t + 1)


def pair_counts(wl) -> Dict[str, int]:
    """Attended (query head, key) pairs per branch for one workload, all batch elements."""
    pos = np.arange(wl.q_start, wl.q_start + wl.q_len, dtype=np.int64)
    vid = (pos >= wl.text_lead) & (pos < wl.kv_len - wl.text_tail)
    tv, tt = pos[vid], pos[~vid]
    H = wl.num_q_heads * wl.batch
    return dict(
        cmp=int(cmp_visible(tv, wl.cmp_block, wl.cmp_stride, wl.kv_len).sum()) * H,
        slc=int(slc_keys(tv, wl.sel_block, wl.top_n).sum()) * H,
        swa=int(swa_keys(tv, wl.window).sum()) * H,
        text=int((tt + 1).sum()) * H,
    )


def flops(wl) -> Dict[str, float]:
    c = pair_counts(wl)
    f = {k: 4.0 * wl.head_dim * v for k, v in c.items()}
    f["total"] = sum(f.values())
    return f


def backward_flops(wl) -> Dict[str, float]:
    """Algorithmic FLOPs of the backward pass: per attended (query head, key) pair the score
    and the upstream product <d_out, v> (recomputed), and the three gradient products dq, dk, dv,
    each 2 D: 10 D per pair (2.5x the forward's 4 D)."""
    c = pair_counts(wl)
    f = {k: 10.0 * wl.head_dim * v for k, v in c.items()}
    f["total"] = sum(f.values())
    return f


def dense_causal_pairs(T: int) -> int:
    """Causal (query, key) pairs of one head over T tokens."""
    return T * (T + 1) // 2
