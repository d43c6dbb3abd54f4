#!/usr/bin/env python
"""Benchmark of the hybrid NSA layer forward pass on one MI355X.

A step is one call of nsa_hybrid_layer_fwd (compression, compression-branch
attention with block importance, top-n, window and text rows, selection branch
with the gated combine) on one batch of synthetic inputs already resident in
HBM.  The headline workload is the 128K-token Qwen2.5-VL-7B-shaped prefill
(tokens/s).  The same run also

* times every phase of the layer with HIP events recorded by the library on its
  own stream (a second, profiled pass over the same steps),
* times the 16 x 64K decode step (GB/s of algorithmic bytes), rotating over
  independent caches so the working set is not served from the last-level cache,
* times the fp64 CPU oracle on a bounded row sample of the same prefill.

Prints one JSON line.  Only N = 1 GPU is supported.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# sources of each timed phase's main kernel (a counter record holds only while they are unchanged)
PHASE_SOURCES = {
    "cmp_attn_importance": ["sparse_attention_long_fwd_amd/csrc/cmp_group.hip",
                            "sparse_attention_long_fwd_amd/csrc/fast_common.hpp",
                            "sparse_attention_long_fwd_amd/csrc/mfma.hpp",
                            "sparse_attention_long_fwd_amd/csrc/common.hpp",
                            "sparse_attention_long_fwd_amd/csrc/api.cpp"],
}
# the kernels of each phase (name fragments); the compression branch runs its first sweep
# (log-sum-exp) and its second sweep (probabilities, value sum, importance) as two kernels
PHASE_KERNELS = {"cmp_attn_importance": ("cmp_lse_kernel", "cmp_group_kernel")}
# one launch of this kernel per layer call and sequence: counts the calls in a counter run
CALL_KERNEL = "compress_kv16_kernel"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
# kernels whose counters the bench line carries: name fragment -> sources
COUNTER_KERNELS = {
    "cmp_lse_kernel": PHASE_SOURCES["cmp_attn_importance"],
    "cmp_group_kernel": PHASE_SOURCES["cmp_attn_importance"],
    "flash_fast_kernel": ["sparse_attention_long_fwd_amd/csrc/flash_fast.hip",
                          "sparse_attention_long_fwd_amd/csrc/fast_common.hpp",
                          "sparse_attention_long_fwd_amd/csrc/mfma.hpp",
                          "sparse_attention_long_fwd_amd/csrc/fast_dispatch.hip"],
    "slc_chunk_kernel": ["sparse_attention_long_fwd_amd/csrc/slc_block.hip",
                         "sparse_attention_long_fwd_amd/csrc/fast_common.hpp"],
    "slc_merge_kernel": ["sparse_attention_long_fwd_amd/csrc/slc_block.hip",
                         "sparse_attention_long_fwd_amd/csrc/fast_common.hpp",
                         "sparse_attention_long_fwd_amd/csrc/fast_dispatch.hip",
                         "sparse_attention_long_fwd_amd/csrc/api.cpp"],
    "dcmp_pipe_kernel": ["sparse_attention_long_fwd_amd/csrc/decode_fast.hip",
                         "sparse_attention_long_fwd_amd/csrc/topk_wave.hpp"],
    "dsel_kernel": ["sparse_attention_long_fwd_amd/csrc/decode_fast.hip",
                    "sparse_attention_long_fwd_amd/csrc/topk_wave.hpp"],
    "gate_proj_kernel": ["sparse_attention_long_fwd_amd/csrc/gate_proj.hip",
                         "sparse_attention_long_fwd_amd/csrc/mfma.hpp"],
}
SIMDS_PER_XCD = 32 * 4  # GRBM_GUI_ACTIVE sums core cycles over the 8 XCDs
COPY_PROBE_BYTES = 1 << 30
PEAK_BF16_MFMA = 2.5e15   # FLOP/s, MI355X dense bf16
PEAK_HBM = 8.0e12         # B/s, MI355X HBM3E
METRIC = "NSA layer prefill tokens/s @128K (MFMA util %); decode GB/s @64K"


def device_clock():
    """The GPU's compute units and shader clock (the runtime's peak clock, and the current one from
    the driver's sysfs table when readable), with the dense bf16 MFMA peak they give at 4,096
    FLOP per cycle and compute unit (2.5 PFLOP/s at 256 units and 2.4 GHz).  The roofline keeps the
    published peak; this records the clock it rests on."""
    import ctypes
    import glob
    out = {}
    try:
        # the HIP runtime this process already runs on (no second copy)
        path = next((ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln), None)
        if path is None:
            return out
        hip = ctypes.CDLL(path)
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0:  # hipDeviceAttributeClockRate, kHz
            out["sclk_peak_mhz"] = v.value / 1000.0
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 63, 0) == 0:  # hipDeviceAttributeMultiprocessorCount
            out["compute_units"] = v.value
    except OSError:
        pass
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for ln in open(f).read().splitlines():
                if ln.strip().endswith("*"):
                    out["sclk_now_mhz"] = float(ln.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
        except (OSError, ValueError, IndexError):
            continue
        if "sclk_now_mhz" in out:
            break
    if "sclk_peak_mhz" in out and "compute_units" in out:
        out["bf16_dense_peak_tflops_from_clock"] = out["compute_units"] * 4096 * out["sclk_peak_mhz"] * 1e6 / 1e12
    return out


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="128k", choices=["128k", "36k", "sweep"])
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    ap.add_argument("--no-prefill", action="store_true", help="decode only (no headline value; for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-phase timing pass")
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--no-gate-proj", action="store_true", help="skip the gate projection measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass measurement (36K)")
    ap.add_argument("--no-budget-sweep", action="store_true",
                    help="skip the fixed-budget (top-n, window) performance surface")
    ap.add_argument("--sweep-steps", type=int, default=5, help="timed steps per budget point")
    ap.add_argument("--no-branch-kv", action="store_true", help="skip the per-branch K/V prefill measurement")
    ap.add_argument("--no-36k", action="store_true", help="skip the 36K prefill measurement")
    ap.add_argument("--no-sweep-runs", action="store_true",
                    help="skip the six 1 %%-text budget / gate runs at 128K")
    ap.add_argument("--varlen-only", action="store_true",
                    help="with --no-prefill: only the variable-length paged decode (for profiling)")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the variable-length paged decode measurement")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run one elementwise copy of 1 GiB (reference for counter runs)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc output directories "
                         "(FETCH_SIZE, then WRITE_SIZE) of a --copy-probe run, and exit")
    ap.add_argument("--record-counters", nargs=3, metavar=("MFMA_DIRS", "EA_READ_DIRS", "EA_WRITE_DIRS"),
                    help="write profiles/counters.json from rocprofv3 --pmc output directories (comma-separated runs) "
                         "(SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA GRBM_GUI_ACTIVE; TCC_EA0_RDREQ_*; "
                         "TCC_EA0_WRREQ_*), and exit")
    return ap.parse_args()


def sources_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def kernel_traffic(phase):
    """HBM bytes per layer call of the phase's kernels, from the committed counter record, or None when
    there is none or the kernels' sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)[phase]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sha256") != sources_sha(rec["sources"]):
        return None
    return rec["bytes_per_call"]


def record_traffic(fetch_dir, write_dir):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each phase's kernels, scaled by what the same
    counter reads for the 1 GiB elementwise copy of --copy-probe, summed over the dispatches of one
    layer call (all row chunks), into profiles/traffic.json."""
    import csv
    import glob

    def read(d, counter):
        path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        per = {}
        for r in rows:  # sum over the counter's instances per dispatch
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        return per

    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = read(d, counter)
        copy = [v for (_, name), v in per.items() if "CUDAFunctor_add" in name or "AddFunctor" in name]
        if not copy:
            raise SystemExit("no copy-probe kernel in %s" % d)
        factor = COPY_PROBE_BYTES / (copy[0] * 1024.0)
        calls = sum(1 for (_, name) in per if CALL_KERNEL in name)
        if calls < 1:
            raise SystemExit("no %s dispatch in %s" % (CALL_KERNEL, d))
        for phase, frags in PHASE_KERNELS.items():
            vals = [v for (_, name), v in per.items() if any(f in name for f in frags)]
            if not vals:
                continue
            rec = out.setdefault(phase, {"kernels": list(frags), "sources": PHASE_SOURCES[phase],
                                         "sha256": sources_sha(PHASE_SOURCES[phase])})
            rec[counter.lower() + "_kib_per_call"] = sum(vals) / calls
            rec[counter.lower() + "_copy_factor"] = factor
            rec["dispatches_per_call"] = len(vals) / calls
    for rec in out.values():
        rec["bytes_per_call"] = (rec["fetch_size_kib_per_call"] * rec["fetch_size_copy_factor"] +
                                 rec["write_size_kib_per_call"] * rec["write_size_copy_factor"]) * 1024.0
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(out))


def record_counters(mfma_dir, ea_r_dir, ea_w_dir):
    """Per-dispatch averages of the matrix-core busy cycles against GPU-active cycles and of the
    L2-to-memory requests (bytes by request size) of the kernels in COUNTER_KERNELS, into
    profiles/counters.json."""
    import csv
    import glob

    def read(dirs):  # comma-separated output directories of separate runs
        per = {}
        for i, d in enumerate(dirs.split(",")):
            path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
            run = {}
            for r in csv.DictReader(open(path)):
                key = (i, int(r["Dispatch_Id"]), r["Kernel_Name"])
                c = run.setdefault(key, {})
                c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            # with more than one layer call in the run, only the last call's dispatches count (the
            # first launch of a kernel in a process carries its start-up in the active cycles)
            calls = sorted(k[1] for k in run if CALL_KERNEL in k[2])
            first = calls[-1] if len(calls) > 1 else -1
            per.update({k: v for k, v in run.items() if k[1] >= first})
        return per

    out = {}
    for frag, srcs in COUNTER_KERNELS.items():
        rec = {"sources": srcs, "sha256": sources_sha(srcs)}
        for d, kind in ((mfma_dir, "mfma"), (ea_r_dir, "read"), (ea_w_dir, "write")):
            vals = [c for (_, _, name), c in read(d).items() if frag in name]
            if not vals:
                continue
            n = len(vals)
            tot = {k: sum(v.get(k, 0.0) for v in vals) / n for k in vals[0]}
            if kind == "mfma":
                rec["mfma_busy_frac"] = tot["SQ_VALU_MFMA_BUSY_CYCLES"] / (tot["GRBM_GUI_ACTIVE"] * SIMDS_PER_XCD)
                rec["mfma_insts"] = tot["SQ_INSTS_MFMA"]
                rec["grbm_gui_active"] = tot["GRBM_GUI_ACTIVE"]
            elif kind == "read":
                rec["mem_read_bytes"] = (32 * tot["TCC_EA0_RDREQ_32B_sum"] + 64 * tot["TCC_EA0_RDREQ_64B_sum"] +
                                         128 * tot["TCC_EA0_RDREQ_128B_sum"])
            else:
                w64 = tot["TCC_EA0_WRREQ_64B_sum"]
                rec["mem_write_bytes"] = 64 * w64 + 32 * (tot["TCC_EA0_WRREQ_sum"] - w64)
            rec["dispatches_" + kind] = n
        if len(rec) > 2:  # counters were found for it
            out[frag] = rec
    with open(COUNTERS_FILE, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(out))


def kernel_counters():
    """Counter record of each kernel whose sources are unchanged since it was taken."""
    try:
        with open(COUNTERS_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    out = {}
    for name, r in rec.items():
        if r.get("sha256") == sources_sha(r["sources"]):
            out[name] = {k: v for k, v in r.items() if k not in ("sources", "sha256")}
    return out or None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def time_calls(fn, reps, stream, per_call=None):
    """Average milliseconds per call of fn() over reps calls, HIP events on `stream`; per_call (a
    list) receives each call's milliseconds from events between the calls."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(reps - 1)] if per_call is not None else []
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(reps):
        fn()
        if i < len(marks):
            marks[i].record(stream)
    end.record(stream)
    end.synchronize()
    if per_call is not None:
        ev = [start] + marks + [end]
        per_call.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
    return start.elapsed_time(end) / reps


def phase_rates(wl, ms):
    """Algorithmic rates per phase: FLOPs for the attention phases, bytes for the rest."""
    from sparse_attention_long_fwd_amd import accounting, nsa

    fl = accounting.flops(wl)
    B, T, Tq, Hq, Hkv, D = wl.batch, wl.kv_len, wl.q_len, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    Nc = nsa.num_cmp_blocks(T, wl.cmp_block, wl.cmp_stride)
    pos = np.arange(wl.q_start, wl.q_start + Tq)
    vid = (pos >= wl.text_lead) & (pos < T - wl.text_tail)
    # compress: read K and V once; write compressed keys (bf16 high part, fp8 low part, a scale byte
    # per 32 channels) and values (bf16 high + low parts)
    b_cmpr = B * (2 * T * Hkv * D * 2 + Nc * Hkv * (D * 3 + D // 32) + 2 * Nc * Hkv * D * 2)
    # top-n: read each video row's candidate importances (blocks 0 .. t / 64), write the chosen blocks
    b_topk = B * Hkv * (int((pos[vid] // wl.sel_block + 1).sum()) * 4 + int(vid.sum()) * wl.top_n * 4)
    # selection: the chosen blocks' K and V, per (video row, group)
    slc_keys = accounting.slc_keys(pos[vid], wl.sel_block, wl.top_n).sum()
    b_slc = B * Hkv * int(slc_keys) * D * 2 * 2
    out = {}
    names = ("compress", "cmp_attn_importance", "topk", "window_text", "selection_combine")
    for name, t in zip(names, ms):
        d = dict(ms=t)
        if name == "compress":
            d.update(bound="hbm", algo_bytes=b_cmpr, gbps=b_cmpr / (t * 1e-3) / 1e9)
        elif name == "topk":
            d.update(bound="hbm", algo_bytes=b_topk, gbps=b_topk / (t * 1e-3) / 1e9)
        elif name == "cmp_attn_importance":
            d.update(bound="mfma", algo_flops=fl["cmp"], tflops=fl["cmp"] / (t * 1e-3) / 1e12)
        elif name == "window_text":
            f = fl["swa"] + fl["text"]
            d.update(bound="mfma", algo_flops=f, tflops=f / (t * 1e-3) / 1e12)
        else:
            # MFMA-bound by definition of the method; block-major, its memory traffic is about
            # 1/5 of the row-major gather of the chosen blocks (reported for context)
            d.update(bound="mfma", algo_flops=fl["slc"], tflops=fl["slc"] / (t * 1e-3) / 1e12,
                     row_major_gather_bytes=b_slc)
        out[name] = d
    return out


def prefill(args, wl, steps=None, warmup=None, inp=None):
    """Time `steps` calls of the layer on `wl` (inputs drawn unless given); the per-phase pass unless
    --no-kernels.  Returns the timing record and the inputs."""
    import torch
    from sparse_attention_long_fwd_amd import accounting, nsa, synth

    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    dev = "cuda"
    stream = torch.cuda.current_stream()
    if inp is None:
        log("generating %s inputs" % wl.name)
        inp = synth.make_inputs(wl, dev)
    q, k, v, g, vid = inp["q"], inp["k"], inp["v"], inp["gates"], inp["is_video"]
    B, Tq, Hq, D = q.shape
    Hkv = k.shape[2]
    sh = nsa.make_shape(B, Tq, wl.kv_len, wl.q_start, Hq, Hkv, D)
    pr = nsa.make_params(**wl.params())
    dt = nsa.NSA_BF16 if wl.dtype == "bf16" else nsa.NSA_F32
    ws = torch.empty(nsa.nsa_hybrid_layer_workspace_size(sh, pr, dt), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)

    def step():
        nsa.nsa_hybrid_layer_fwd(q, k, v, g, sh, pr, w_k=inp["w_k"], w_v=inp["w_v"], is_video=vid, out=out,
                                 workspace=ws, stream=stream)

    log("%s: warmup %d" % (wl.name, warmup))
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log("%s: timing %d steps" % (wl.name, steps))
    t0 = time.perf_counter()
    each = []
    ms = time_calls(step, steps, stream, each)
    wall = time.perf_counter() - t0
    fl = accounting.flops(wl)
    res = dict(workload=wl.name, steps=steps, ms_per_step=ms, ms_median=float(np.median(each)),
               ms_min=float(np.min(each)), wall_s=wall, tokens_per_s=wl.q_len * wl.batch / (ms * 1e-3),
               algo_flops=fl, algo_tflops=fl["total"] / (ms * 1e-3) / 1e12,
               mfma_util=fl["total"] / (ms * 1e-3) / PEAK_BF16_MFMA)
    if not args.no_kernels:
        log("%s: per-phase timing (%d steps)" % (wl.name, steps))
        nsa.profile_enable(True)
        acc = None
        for _ in range(steps):
            step()
            ph = np.array(nsa.profile_read())
            acc = ph if acc is None else acc + ph
        nsa.profile_enable(False)
        res["kernels"] = phase_rates(wl, list(acc / steps))
    del ws
    return res, inp


def branch_outputs(wl, inp):
    """One more layer call (untimed) that also returns the branch outputs and the chosen blocks,
    for the parity statistics of the CPU-baseline leg."""
    import torch
    from sparse_attention_long_fwd_amd import nsa

    q, k = inp["q"], inp["k"]
    B, Tq, Hq, D = q.shape
    sh = nsa.make_shape(B, Tq, wl.kv_len, wl.q_start, Hq, k.shape[2], D)
    pr = nsa.make_params(**wl.params())
    got = dict(o_cmp=torch.empty_like(q), o_slc=torch.empty_like(q), o_swa=torch.empty_like(q),
               idx=torch.full((B, Tq, k.shape[2], wl.top_n), -1, dtype=torch.int32, device=q.device))
    got["out"] = nsa.nsa_hybrid_layer_fwd(q, k, inp["v"], inp["gates"], sh, pr, w_k=inp["w_k"], w_v=inp["w_v"],
                                          is_video=inp["is_video"], o_cmp=got["o_cmp"], o_slc=got["o_slc"],
                                          o_swa=got["o_swa"], block_idx_out=got["idx"])
    torch.cuda.synchronize()
    return got


BUDGET = 16 * 64 + 512   # tokens each video row attends in the selection + window branches
# (selection block l', top-n, window) with l' n + w = BUDGET
BUDGET_POINTS = [(64, 8, 1024), (64, 12, 768), (64, 16, 512), (64, 20, 256), (64, 22, 128), (64, 23, 64),
                 (32, 24, 768), (32, 32, 512), (128, 8, 512), (128, 10, 256)]


def budget_sweep(args, wl, inp):
    """Performance surface of the selection / window split at a fixed budget: top-n blocks of l'
    tokens plus a window of w tokens with l' n + w = 1536 (l' = 32, 64, 128), on the same 128K
    inputs; per point the step time, tokens/s, algorithmic FLOP rate and the library's phase
    times."""
    import torch
    from sparse_attention_long_fwd_amd import accounting, nsa

    stream = torch.cuda.current_stream()
    q, k, v, g, vid = inp["q"], inp["k"], inp["v"], inp["gates"], inp["is_video"]
    B, Tq, Hq, D = q.shape
    sh = nsa.make_shape(B, Tq, wl.kv_len, wl.q_start, Hq, k.shape[2], D)
    out = torch.empty_like(q)
    pts = []
    for ls, n, w in BUDGET_POINTS:
        assert ls * n + w == BUDGET
        wv = wl.with_(sel_block=ls, top_n=n, window=w)
        pr = nsa.make_params(**wv.params())
        ws = torch.empty(nsa.nsa_hybrid_layer_workspace_size(sh, pr, nsa.NSA_BF16), dtype=torch.uint8,
                         device="cuda")

        def step():
            nsa.nsa_hybrid_layer_fwd(q, k, v, g, sh, pr, w_k=inp["w_k"], w_v=inp["w_v"], is_video=vid, out=out,
                                     workspace=ws, stream=stream)

        for _ in range(2):
            step()
        ms = time_calls(step, args.sweep_steps, stream)
        nsa.profile_enable(True)
        acc = None
        for _ in range(args.sweep_steps):
            step()
            ph = np.array(nsa.profile_read())
            acc = ph if acc is None else acc + ph
        nsa.profile_enable(False)
        fl = accounting.flops(wv)["total"]
        pts.append(dict(sel_block=ls, top_n=n, window=w, ms_per_step=ms, tokens_per_s=Tq * B / (ms * 1e-3),
                        algo_tflops=fl / (ms * 1e-3) / 1e12,
                        phase_ms={name: round(float(x), 4) for name, x in zip(nsa.PHASES, acc / args.sweep_steps)}))
        log("budget point l'=%d n=%d w=%d: %.2f ms" % (ls, n, w, ms))
        del ws
    return dict(workload=wl.name, budget_tokens=BUDGET, points=pts)


def branch_kv(args, wl, inp):
    """The same 128K prefill with independent keys / values per branch (compression, selection,
    window + text rows): three K/V pairs in HBM, the same kernels."""
    import torch
    from sparse_attention_long_fwd_amd import nsa, synth

    stream = torch.cuda.current_stream()
    kv = {}
    for tag, off in (("s", 40), ("w", 80)):
        other = synth.make_inputs(wl, "cuda", batch_offset=off)
        kv[tag] = (other["k"], other["v"])
        del other
    q = inp["q"]
    B, Tq, Hq, D = q.shape
    sh = nsa.make_shape(B, Tq, wl.kv_len, wl.q_start, Hq, inp["k"].shape[2], D)
    pr = nsa.make_params(**wl.params())
    ws = torch.empty(nsa.nsa_hybrid_layer_workspace_size(sh, pr, nsa.NSA_BF16), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)

    def step():
        nsa.nsa_hybrid_layer_fwd_branch_kv(q, (inp["k"], inp["v"]), kv["s"], kv["w"], inp["gates"], sh, pr,
                                           w_k=inp["w_k"], w_v=inp["w_v"], is_video=inp["is_video"], out=out,
                                           workspace=ws, stream=stream)

    for _ in range(2):
        step()
    ms = time_calls(step, args.sweep_steps, stream)
    del ws, kv
    return dict(workload=wl.name, ms_per_step=ms, tokens_per_s=Tq * B / (ms * 1e-3), steps=args.sweep_steps)


def backward(args):
    """Backward pass of the 36K layer (the matrix-core kernels; the generic VALU kernels timed once
    beside them): gradients of sum(d_out * out) for q, k, v, the gates and the compression weights,
    the forward's chosen blocks held fixed."""
    import torch
    from sparse_attention_long_fwd_amd import accounting, nsa, synth

    wl = synth.WORKLOADS["36k"]
    stream = torch.cuda.current_stream()
    inp = synth.make_inputs(wl, "cuda")
    B, Tq, Hq, D = inp["q"].shape
    sh = nsa.make_shape(B, Tq, wl.kv_len, wl.q_start, Hq, wl.num_kv_heads, D)
    pr = nsa.make_params(**wl.params())
    idx = torch.full((B, Tq, wl.num_kv_heads, wl.top_n), -1, dtype=torch.int32, device="cuda")
    nsa.nsa_hybrid_layer_fwd(inp["q"], inp["k"], inp["v"], inp["gates"], sh, pr, w_k=inp["w_k"], w_v=inp["w_v"],
                             is_video=inp["is_video"], block_idx_out=idx, stream=stream)
    dout = synth.normal(1000 * wl.index + 900, (B, Tq, Hq, D), "cuda").to(torch.bfloat16)
    ws = torch.empty(nsa.nsa_hybrid_layer_bwd_workspace_size(sh, pr, nsa.NSA_BF16), dtype=torch.uint8,
                     device="cuda")

    def step():
        nsa.nsa_hybrid_layer_bwd(inp["q"], inp["k"], inp["v"], inp["gates"], idx, dout, sh, pr, w_k=inp["w_k"],
                                 w_v=inp["w_v"], is_video=inp["is_video"], workspace=ws, stream=stream)

    step()
    steps = 5
    ms = time_calls(step, steps, stream)
    prev = nsa.set_force_generic(True)
    try:
        ws = torch.empty(nsa.nsa_hybrid_layer_bwd_workspace_size(sh, pr, nsa.NSA_BF16), dtype=torch.uint8,
                         device="cuda")
        ms_generic = time_calls(step, 1, stream)
    finally:
        nsa.set_force_generic(prev)
    fl = accounting.backward_flops(wl)["total"]
    del inp, ws
    return dict(workload=wl.name, kernels="matrix cores (bf16 MFMA)", ms_per_step=ms, algo_flops=fl,
                tflops=fl / (ms * 1e-3) / 1e12, mfma_frac=fl / (ms * 1e-3) / PEAK_BF16_MFMA, steps=steps,
                ms_generic_kernels=ms_generic)


def decode(args):
    """16 x 64K decode step, rotating over 4 independent caches."""
    import torch
    from sparse_attention_long_fwd_amd import nsa, synth

    wl = synth.WORKLOADS["decode"]
    dev = "cuda"
    stream = torch.cuda.current_stream()
    sets = []
    n_rot = 4
    for r in range(n_rot):
        log("decode cache %d" % r)
        inp = synth.make_inputs(wl, dev, batch_offset=wl.batch * r)
        kc, vc = nsa.nsa_compress_kv(inp["k"], inp["v"], inp["w_k"], inp["w_v"], wl.cmp_block, wl.cmp_stride)
        inp["kc"], inp["vc"] = kc, vc
        sets.append(inp)
    q0 = sets[0]["q"]
    B, Tq, Hq, D = q0.shape
    Hkv = sets[0]["k"].shape[2]
    sh = nsa.make_shape(B, Tq, wl.kv_len, wl.q_start, Hq, Hkv, D)
    pr = nsa.make_params(**wl.params())
    ws = torch.empty(nsa.nsa_hybrid_layer_workspace_size(sh, pr, nsa.NSA_BF16), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(s["q"]) for s in sets]
    idxs = [torch.full((B, Tq, Hkv, wl.top_n), -1, dtype=torch.int32, device=dev) for _ in sets]
    state = {"i": 0}

    def step():
        i = state["i"] % n_rot
        s = sets[i]
        nsa.nsa_hybrid_layer_fwd(s["q"], s["k"], s["v"], s["gates"], sh, pr, k_cmp_in=s["kc"], v_cmp_in=s["vc"],
                                 is_video=s["is_video"], out=outs[i], block_idx_out=idxs[i], workspace=ws,
                                 stream=stream)
        state["i"] += 1

    for _ in range(2 * n_rot):
        step()
    ms = time_calls(step, args.decode_steps, stream)
    # the same steps captured once per cache into HIP graphs and replayed in rotation
    ms_graph = None
    try:
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for i in range(n_rot):
                gph = torch.cuda.CUDAGraph()
                state["i"] = i
                with torch.cuda.graph(gph, stream=cap):
                    s = sets[i]
                    nsa.nsa_hybrid_layer_fwd(s["q"], s["k"], s["v"], s["gates"], sh, pr, k_cmp_in=s["kc"],
                                             v_cmp_in=s["vc"], is_video=s["is_video"], out=outs[i],
                                             block_idx_out=idxs[i], workspace=ws, stream=cap)
                graphs.append(gph)
        torch.cuda.current_stream().wait_stream(cap)
        gstate = {"i": 0}

        def replay():
            graphs[gstate["i"] % n_rot].replay()
            gstate["i"] += 1

        for _ in range(2 * n_rot):
            replay()
        ms_graph = time_calls(replay, args.decode_steps, torch.cuda.current_stream())
    except Exception as exc:  # report, keep the plain-launch number
        log("graph capture of the decode step failed: %s" % exc)
    # algorithmic bytes: compressed cache + the union of selected-block and window tokens, each once,
    # plus q, out and gates
    t = wl.q_start
    Nc = nsa.num_cmp_blocks(wl.kv_len, wl.cmp_block, wl.cmp_stride)
    total = 0
    for i in range(n_rot):
        idx = idxs[i].cpu().numpy()
        for b in range(B):
            for g in range(Hkv):
                toks = set(range(max(0, t - wl.window + 1), t + 1))
                for j in idx[b, 0, g]:
                    if j >= 0:
                        toks |= set(range(j * wl.sel_block, min((j + 1) * wl.sel_block, t + 1)))
                total += (2 * Nc + 2 * len(toks)) * D * 2
    total = total / n_rot + B * Hq * D * 2 * 2 + B * Hq * 3 * 4
    bw = total / (ms * 1e-3)
    bw_g = total / (ms_graph * 1e-3) if ms_graph else None
    return dict(workload=wl.name, ms_per_step=ms, algo_bytes=total, gbps=bw / 1e9, hbm_frac=bw / PEAK_HBM,
                ms_per_step_graph=ms_graph, gbps_graph=bw_g / 1e9 if bw_g else None,
                hbm_frac_graph=bw_g / PEAK_HBM if bw_g else None, rotating_caches=n_rot, steps=args.decode_steps,
                roofline=dict(bound="hbm", achieved=bw / 1e9, peak=PEAK_HBM / 1e9, unit="GB/s", frac=bw / PEAK_HBM))


def decode_varlen(args):
    """Variable-length decode over a paged cache: 16 sequences of 4K..64K tokens (seeded), pages of 64
    tokens at shuffled pool positions; a step is the compressed-cache update for one appended token
    plus the decode row of every sequence.  Rotates over 4 independent pools."""
    import torch
    from sparse_attention_long_fwd_amd import nsa, synth

    wl = synth.WORKLOADS["decode_varlen"]
    lens = synth.decode_lengths(wl)
    dev = "cuda"
    stream = torch.cuda.current_stream()
    B, T, Hkv, D = wl.batch, wl.kv_len, wl.num_kv_heads, wl.head_dim
    mp = T // nsa.PAGE_ROWS
    lens_t = torch.tensor(lens, dtype=torch.int32, device=dev)
    sets = []
    n_rot = 4
    for r in range(n_rot):
        log("decode_varlen pool %d" % r)
        inp = synth.make_inputs(wl, dev, batch_offset=wl.batch * r)
        gen = torch.Generator().manual_seed(1000 * wl.index + r)
        perm = torch.randperm(B * mp, generator=gen).to(dev)
        s = dict(q=inp["q"], gates=inp["gates"], is_video=inp["is_video"], table=perm.view(B, mp).to(torch.int32))
        for name in ("k", "v"):
            pool = torch.empty(B * mp, nsa.PAGE_ROWS, Hkv, D, dtype=inp[name].dtype, device=dev)
            pool[perm] = inp[name].view(B * mp, nsa.PAGE_ROWS, Hkv, D)
            s[name] = pool
            del inp[name]
        Nc = nsa.num_cmp_blocks(T, wl.cmp_block, wl.cmp_stride)
        s["kc"] = torch.zeros(B, Nc, Hkv, D, dtype=torch.bfloat16, device=dev)
        s["vc"] = torch.zeros_like(s["kc"])
        nsa.nsa_compress_append(s["k"], s["v"], inp["w_k"], inp["w_v"], s["kc"], s["vc"], T, T, kv_lens=lens_t,
                                page_table=s["table"])
        s["w_k"], s["w_v"] = inp["w_k"], inp["w_v"]
        sets.append(s)
    Hq = sets[0]["q"].shape[2]
    sh = nsa.make_shape(B, 1, T, 0, Hq, Hkv, D)
    pr = nsa.make_params(**wl.params())
    ws = torch.empty(nsa.nsa_decode_workspace_size(sh, pr, nsa.NSA_BF16), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(s["q"]) for s in sets]
    idxs = [torch.full((B, 1, Hkv, wl.top_n), -1, dtype=torch.int32, device=dev) for _ in sets]
    state = {"i": 0}

    def step():
        i = state["i"] % n_rot
        s = sets[i]
        nsa.nsa_compress_append(s["k"], s["v"], s["w_k"], s["w_v"], s["kc"], s["vc"], T, 1, kv_lens=lens_t,
                                page_table=s["table"], stream=stream)
        nsa.nsa_decode_fwd(s["q"], s["k"], s["v"], s["kc"], s["vc"], s["gates"], sh, pr, kv_lens=lens_t,
                           page_table=s["table"], is_video=s["is_video"], out=outs[i], block_idx_out=idxs[i],
                           workspace=ws, stream=stream)
        state["i"] += 1

    for _ in range(2 * n_rot):
        step()
    ms = time_calls(step, args.decode_steps, stream)
    # algorithmic bytes per sequence: its visible compressed blocks, the union of its selected-block and
    # window tokens, each once, the appended block's l tokens when the new token completes one; plus q,
    # out and gates
    total = 0
    for i in range(n_rot):
        idx = idxs[i].cpu().numpy()
        for b, L in enumerate(lens):
            t = L - 1
            nc = nsa.num_cmp_blocks(L, wl.cmp_block, wl.cmp_stride)
            app = (L - wl.cmp_block) >= 0 and (L - wl.cmp_block) % wl.cmp_stride == 0
            for g in range(Hkv):
                toks = set(range(max(0, t - wl.window + 1), t + 1))
                for j in idx[b, 0, g]:
                    if j >= 0:
                        toks |= set(range(j * wl.sel_block, min((j + 1) * wl.sel_block, t + 1)))
                total += (2 * nc + 2 * len(toks)) * D * 2
                if app:
                    total += (2 * wl.cmp_block * D * 2 + 2 * D * 2)
    total = total / n_rot + B * Hq * D * 2 * 2 + B * Hq * 3 * 4
    bw = total / (ms * 1e-3)
    return dict(workload=wl.name, lens_min=min(lens), lens_max=max(lens), lens_mean=float(np.mean(lens)),
                page_rows=nsa.PAGE_ROWS, ms_per_step=ms, algo_bytes=total, gbps=bw / 1e9, hbm_frac=bw / PEAK_HBM,
                rotating_pools=n_rot, steps=args.decode_steps)


def gate_proj(args, wl):
    """Gate projection in front of the layer: sigmoid(x w_g^T + b) for every token of the workload,
    x [1, T, 3584] bf16 hidden states (Qwen2.5-VL-7B), w_g [3 Hq, 3584]; HBM-bound on x."""
    import torch
    from sparse_attention_long_fwd_amd import nsa, synth

    gi = synth.make_gate_inputs(wl, "cuda")
    g = torch.empty(wl.batch, wl.q_len, wl.num_q_heads, 3, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        nsa.nsa_gate_proj(gi["x"], gi["w_g"], gi["b_g"], gates=g, stream=stream)

    for _ in range(3):
        step()
    ms = time_calls(step, max(20, args.steps), stream)
    byts = gi["x"].numel() * 2 + gi["w_g"].numel() * 2 + gi["b_g"].numel() * 4 + g.numel() * 4
    flops = 2.0 * gi["x"].numel() * gi["w_g"].shape[0]
    bw = byts / (ms * 1e-3)
    del gi, g
    return dict(workload="%s hidden=%d" % (wl.name, synth.HIDDEN), ms_per_call=ms, algo_bytes=byts,
                gbps=bw / 1e9, hbm_frac=bw / PEAK_HBM, tflops=flops / (ms * 1e-3) / 1e12,
                roofline=dict(bound="hbm", achieved=bw / 1e9, peak=PEAK_HBM / 1e9, unit="GB/s", frac=bw / PEAK_HBM))


def _host(t):
    import torch
    return (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy()


def cpu_sample_rows(wl, seed):
    """The oracle's row sample of a prefill: one video row per 64-token frame at a seeded offset
    inside the frame, every text row, and the first and last 1,024 rows."""
    T = wl.q_len
    rng = np.random.default_rng(seed)
    off = int(rng.integers(0, wl.frame))
    pos = np.arange(wl.q_start, wl.q_start + T)
    vid = (pos >= wl.text_lead) & (pos < wl.kv_len - wl.text_tail)
    rows = set(np.nonzero(~vid)[0].tolist())
    rows |= set(range(min(1024, T))) | set(range(max(0, T - 1024), T))
    rows |= set((np.arange(wl.text_lead + off, wl.kv_len - wl.text_tail, wl.frame) - wl.q_start).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < T), dtype=np.int64)


def cpu_baseline_parity(wl, inp, got, rows, ref):
    """Parity of the GPU's layer outputs against the oracle's on the sampled rows (CPU-baseline leg):
    max-abs error per branch and of the output, and the selection statistics of the index rule --
    chosen blocks identical wherever the oracle's gap exceeds 1e-3; where they differ (undecided
    rows) the selection and final outputs are compared against the oracle run on the GPU's set."""
    import oracle

    import torch

    q = _host(inp["q"][0])
    k, v = _host(inp["k"][0]), _host(inp["v"][0])
    vid = _host(inp["is_video"][0])[rows].astype(bool)
    sel = torch.from_numpy(rows).to(inp["q"].device)
    # the GPU's outputs on the sampled rows only (gathered on the device)
    gr = {key: _host(t[0].index_select(0, sel)) for key, t in got.items()}
    gidx = gr["idx"]
    st = dict(rows=int(len(rows)), video_rows=int(vid.sum()))
    err = {}
    if vid.any():
        same = np.all(gidx[vid] == ref["idx"][vid], axis=-1)
        dec = ref["gap"][vid] > 1e-3
        st.update(row_groups=int(same.size), decided=int(dec.sum()), decided_frac=float(dec.mean()),
                  idx_equal_frac=float(same.mean()), decided_mismatches=int((dec & ~same).sum()),
                  substituted_rows=int((~same.all(axis=1)).sum()))
        ref_slc, ref_out = ref["o_slc"][vid].copy(), ref["out"][vid].copy()
        sub = np.nonzero(~same.all(axis=1))[0]
        if sub.size:
            vr = rows[vid][sub]
            o_sub, _ = oracle.sparse_rows(q[vr], vr + wl.q_start, k, v, gidx[vid][sub], wl.sel_block, wl.window,
                                          oracle.default_scale(wl.head_dim), swa=False)
            gg = _host(inp["gates"][0])[vr].astype(np.float64)
            ref_slc[sub] = o_sub
            ref_out[sub] = (gg[..., 0:1] * ref["o_cmp"][vid][sub] + gg[..., 1:2] * o_sub +
                            gg[..., 2:3] * ref["o_swa"][vid][sub])
        for name, r in (("cmp", ref["o_cmp"][vid]), ("swa", ref["o_swa"][vid]), ("slc", ref_slc)):
            err[name] = float(np.max(np.abs(gr["o_" + name][vid] - r)))
        err["out"] = float(np.max(np.abs(gr["out"][vid] - ref_out)))
    if (~vid).any():
        err["text"] = float(np.max(np.abs(gr["out"][~vid] - ref["out"][~vid])))
    st["max_abs"] = err
    tol = 2e-2 if wl.dtype == "bf16" else 1e-4
    st["tolerance"] = tol
    st["pass"] = bool(all(x <= tol for x in err.values()) and st.get("decided_mismatches", 0) == 0)
    return st


def cpu_info():
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def cpu_baseline(args, wl, inp, got):
    """The fp64 oracle on the stated row sample of the same prefill (rank 0), timed on the host's
    cores; the same run checks the GPU's outputs on those rows against it."""
    import oracle
    from sparse_attention_long_fwd_amd import accounting

    rows = cpu_sample_rows(wl, wl.index)
    q = _host(inp["q"][0])
    k, v = _host(inp["k"][0]), _host(inp["v"][0])
    oracle.build()
    t0 = time.perf_counter()
    ref = oracle.layer(q, k, v, _host(inp["w_k"]), _host(inp["w_v"]), _host(inp["gates"][0]),
                       _host(inp["is_video"][0]), wl.params(), q_start=wl.q_start, rows=rows)
    dt = time.perf_counter() - t0
    # extrapolation to the whole layer by the algorithmic work of the rows (compression included)
    pos = np.arange(wl.q_start, wl.q_start + wl.q_len)
    vid = (pos >= wl.text_lead) & (pos < wl.kv_len - wl.text_tail)

    def work(p, v_):
        c = accounting.cmp_visible(p, wl.cmp_block, wl.cmp_stride, wl.kv_len)
        sel = accounting.slc_keys(p, wl.sel_block, wl.top_n)
        swa = accounting.swa_keys(p, wl.window)
        return float(np.where(v_, c + sel + swa, p + 1).sum())

    frac = work(pos[rows], vid[rows]) / work(pos, vid)
    model, visible = cpu_info()
    parity = cpu_baseline_parity(wl, inp, got, rows, ref)
    return dict(value=len(rows) / dt, unit="query rows/s over the sample (extrapolated to the layer: see "
                "extrapolated_layer_s)", cores=oracle.num_threads(), cores_visible=visible, cpu_model=model,
                kind="oracle", seconds=dt, extrapolated=True, extrapolated_layer_s=dt / frac,
                extrapolated_tokens_per_s=wl.q_len / (dt / frac),
                sample="%d rows of the %d-row %s prefill: one video row per 64-token frame at a seeded offset, "
                       "all %d text rows, the first and last 1024 rows (%.2f %% of the layer's attended pairs); "
                       "compression of the whole sequence included" % (
                           len(rows), wl.q_len, wl.name, int((~vid).sum()), 100 * frac),
                parity=parity)


def sampled_rows(wl, n_video, seed, text=4, edge=16):
    """A small seeded row sample for the parity of the secondary runs: evenly spaced video rows at a
    seeded offset, a few text rows from each end, the first and last rows."""
    T = wl.q_len
    rng = np.random.default_rng(seed)
    stride = max(1, (T - wl.text_lead - wl.text_tail) // n_video)
    off = int(rng.integers(0, stride))
    rows = set(range(wl.text_lead + off, T - wl.text_tail, stride))
    rows |= set(range(edge)) | set(range(T - edge, T))
    rows |= set(range(wl.text_lead, wl.text_lead + text // 2)) | set(range(T - wl.text_tail - text // 2,
                                                                            T - wl.text_tail))
    if wl.text_lead:
        rows |= set(range(wl.text_lead - text // 2, wl.text_lead))
    if wl.text_tail:
        rows |= set(range(T - wl.text_tail, T - wl.text_tail + text // 2))
    return np.array(sorted(r for r in rows if 0 <= r < T), dtype=np.int64)


def cpu_baseline_run_parity(wl, inp, n_video, seed):
    """CPU-baseline leg of a secondary prefill run: the oracle on a small row sample and the parity
    statistics of the GPU's outputs there."""
    import oracle

    got = branch_outputs(wl, inp)
    rows = sampled_rows(wl, n_video, seed)
    ref = oracle.layer(_host(inp["q"][0]), _host(inp["k"][0]), _host(inp["v"][0]), _host(inp["w_k"]),
                       _host(inp["w_v"]), _host(inp["gates"][0]), _host(inp["is_video"][0]), wl.params(),
                       q_start=wl.q_start, rows=rows)
    st = cpu_baseline_parity(wl, inp, got, rows, ref)
    del got
    return st


def prefill_36k(args):
    """The 36K-token Qwen2.5-VL-7B-shaped prefill (560 frames + 512 text tokens): throughput and
    algorithmic MFMA rate, and its parity on sampled rows (CPU-baseline leg)."""
    import torch
    from sparse_attention_long_fwd_amd import synth

    wl = synth.WORKLOADS["36k"]
    res, inp = prefill(args, wl, steps=max(10, args.steps), warmup=2)
    if not args.no_cpu_baseline:
        res["parity"] = cpu_baseline_run_parity(wl, inp, 256, wl.index)
    del inp
    torch.cuda.empty_cache()
    return res


def sweep_runs(args):
    """The six 128K runs with 1 % text (640 + 2,028 frames x 64 + 640 tokens): budget (top-n, window)
    in {(16, 512), (8, 256)} x gates {sigmoid(N(0,1)), CMP-dominant, SLC-dominant}; tokens/s and
    algorithmic TFLOP/s each, and parity on sampled rows (CPU-baseline leg)."""
    import torch
    from sparse_attention_long_fwd_amd import synth

    base = synth.WORKLOADS["sweep"]
    inp = synth.make_inputs(base, "cuda")  # gates sigmoid(N(0,1)); q, k, v are the same in every run
    g_sig = inp["gates"]
    out = []
    for i, (n, w, gates) in enumerate(synth.SWEEP_VARIANTS):
        wl = base.with_(top_n=n, window=w, gates=gates)
        if gates == "sigmoid":
            inp["gates"] = g_sig
        else:  # the fixed regime of every (row, head), as make_inputs draws it
            inp["gates"] = torch.tensor(synth.GATE_REGIMES[gates], dtype=torch.float32,
                                        device="cuda").expand_as(g_sig).contiguous()
        res, _ = prefill(args, wl, steps=args.sweep_steps, warmup=2, inp=inp)
        rec = dict(top_n=n, window=w, gates=gates, ms_per_step=res["ms_per_step"], tokens_per_s=res["tokens_per_s"],
                   algo_tflops=res["algo_tflops"], mfma_util=res["mfma_util"])
        if "kernels" in res:
            rec["phase_ms"] = {k: round(v["ms"], 4) for k, v in res["kernels"].items()}
        if not args.no_cpu_baseline:
            rec["parity"] = cpu_baseline_run_parity(wl, inp, 96, i)
        log("sweep n=%d w=%d gates=%s: %.2f ms" % (n, w, gates, res["ms_per_step"]))
        out.append(rec)
    del inp
    torch.cuda.empty_cache()
    return dict(workload=base.name, text_tokens=base.text_lead + base.text_tail, runs=out)


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.record_counters:
        record_counters(*args.record_counters)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the layer would shard by GQA group (up to 4 ways) and then by "
              "query rows, but no multi-GPU path is built; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_attention_long_fwd_amd import nsa, synth

    nsa.lib()
    torch.cuda.init()
    if args.copy_probe:
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.add(src, 0.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    wl = synth.WORKLOADS[args.workload]
    if args.no_prefill:
        res = {} if args.varlen_only else {"decode": decode(args)}
        if not args.no_varlen:
            res["decode_varlen"] = decode_varlen(args)
        print(json.dumps(res))
        return
    res, inp = prefill(args, wl)
    got = None if args.no_cpu_baseline else branch_outputs(wl, inp)
    ker = res.get("kernels", {})
    roofline = None
    if ker:
        dom_name = max(ker, key=lambda n: ker[n]["ms"])
        dom = ker[dom_name]
        if dom["bound"] == "hbm":
            roofline = dict(kernel=dom_name, bound="hbm", achieved=dom["gbps"], peak=PEAK_HBM / 1e9, unit="GB/s",
                            frac=dom["gbps"] * 1e9 / PEAK_HBM, traffic=kernel_traffic(dom_name))
        else:
            roofline = dict(kernel=dom_name, bound="mfma", achieved=dom["tflops"], peak=PEAK_BF16_MFMA / 1e12,
                            unit="TFLOP/s", frac=dom["tflops"] * 1e12 / PEAK_BF16_MFMA,
                            traffic=kernel_traffic(dom_name))
    sweep = None
    if not args.no_budget_sweep and wl.name == synth.WORKLOADS["128k"].name:
        log("budget sweep")
        sweep = budget_sweep(args, wl, inp)
    bkv = None
    if not args.no_branch_kv:
        log("keys / values per branch")
        bkv = branch_kv(args, wl, inp)
    cpu = None
    if not args.no_cpu_baseline:
        log("oracle timing and parity on the sampled rows")
        cpu = cpu_baseline(args, wl, inp, got)
    del inp, got
    torch.cuda.empty_cache()
    p36 = None
    if not args.no_36k and wl.name == synth.WORKLOADS["128k"].name:
        log("36K prefill")
        p36 = prefill_36k(args)
    sw5 = None
    if not args.no_sweep_runs and wl.name == synth.WORKLOADS["128k"].name:
        log("budget / gate runs (1 % text)")
        sw5 = sweep_runs(args)
    gp = None
    if not args.no_gate_proj:
        log("gate projection")
        gp = gate_proj(args, wl)
        torch.cuda.empty_cache()
    bwd = None
    if not args.no_backward:
        log("backward (36K)")
        bwd = backward(args)
        torch.cuda.empty_cache()
    dec = None
    if not args.no_decode:
        log("decode")
        dec = decode(args)
        if not args.no_varlen:
            log("decode_varlen")
            dec["varlen_paged"] = decode_varlen(args)
    line = {
        "metric": METRIC,
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "ms_median": res["ms_median"],
        "ms_min": res["ms_min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64 + Box-Muller; frame-correlated video K; no trained weights)",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.kv_len, "q_heads": wl.num_q_heads,
                   "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "top_n": wl.top_n, "window": wl.window,
                   "cmp_block": wl.cmp_block, "cmp_stride": wl.cmp_stride, "sel_block": wl.sel_block,
                   "text_tokens": wl.text_lead + wl.text_tail, "parallelism": "single GPU"},
        "mfma_util_algorithmic": res["mfma_util"],
        "algo_flops": res["algo_flops"],
        "kernels": ker,
        "roofline": roofline,
        "decode": dec,
        "gate_proj": gp,
        "backward": bwd,
        "budget_sweep": sweep,
        "branch_kv": bkv,
        "prefill_36k": p36,
        "budget_gate_runs": sw5,
        "cpu_baseline": cpu,
        "counters": kernel_counters(),
        "device": device_clock(),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
