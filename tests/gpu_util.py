"""Helpers shared by the GPU parity tests: host copies, oracle runs and the
comparison rules (tolerances and the index gap rule)."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# Output tolerances (max-abs error) by input dtype.
TOL = {"f32": 1e-4, "bf16": 2e-2}
# Chosen blocks must match exactly where the oracle's last-taken and first-left
# free candidates differ by more than this.
GAP = 1e-3


def host(t: torch.Tensor) -> np.ndarray:
    """Exact float32 (or int) host copy of a device tensor."""
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.detach().cpu().numpy()


def flush(msg: str):
    print(msg, flush=True)


def maxabs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def check_indices(gpu_idx, ref_idx, ref_gap, ref_imp, pos, ls, n, n_init, n_local):
    """Index rule.  Returns a bool mask [R, Hkv] of rows whose sets are identical.

    Where the oracle's gap exceeds GAP the sets must be identical.  Everywhere
    else the GPU set must be a valid selection: ascending, -1 padded, the forced
    blocks present, the right size, every free pick within GAP of the oracle's
    last taken free candidate, and every free candidate that lies more than GAP
    above that last taken value taken (a set that drops a clearly better block
    for one inside the band is a mis-ranking, not a tie).
    """
    gpu_idx = np.asarray(gpu_idx)
    same = np.all(gpu_idx == ref_idx, axis=-1)
    must = ref_gap > GAP
    bad = must & ~same
    assert not bad.any(), "index mismatch on %d decided (row, group) pairs, first %s" % (
        bad.sum(), np.argwhere(bad)[:3].tolist())
    for r, g in np.argwhere(~same):
        t = int(pos[r])
        jt = t // ls
        sel = [int(x) for x in gpu_idx[r, g] if x >= 0]
        assert sel == sorted(sel) and len(set(sel)) == len(sel)
        assert all(0 <= x <= jt for x in sel)
        assert len(sel) == min(n, jt + 1)
        assert list(gpu_idx[r, g][len(sel):]) == [-1] * (n - len(sel))
        forced = {j for j in range(jt + 1) if j < n_init or j > jt - n_local}
        assert forced <= set(sel)
        ref_free = [int(x) for x in ref_idx[r, g] if x >= 0 and int(x) not in forced]
        kth = min(ref_imp[r, g, j] for j in ref_free) if ref_free else np.inf
        for x in sel:
            if x not in forced:
                assert ref_imp[r, g, x] >= kth - GAP, (r, g, x)
        clear = set(np.nonzero(np.asarray(ref_imp[r, g, :jt + 1]) > kth + GAP)[0].tolist()) - forced
        missing = clear - set(sel)
        assert not missing, "row %d group %d leaves out blocks %s scored clearly above the band" % (
            r, g, sorted(missing))
    return same
