"""Seeded synthetic inputs for the hybrid NSA layer.

This module holds no part of the attention method's arithmetic.  It only draws
numbers and lays out the workloads (shapes, text/video row layout, parameter
values), so that the GPU path's tests and benchmark and the CPU oracle's tests
consume identical inputs.

Random numbers
--------------
* Uniform 64-bit words come from SplitMix64 (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014), used as a
  counter-based generator: draw ``c`` (0-based) of stream ``seed`` is the mixing
  function applied to ``seed + (c + 1) * 0x9E3779B97F4A7C15 (mod 2**64)``, which
  is exactly the c-th output of a SplitMix64 generator seeded with ``seed``.
* Uniforms in (0, 1] are ``((z >> 11) + 1) * 2**-53``.
* Normals come from the Box-Muller transform (Box and Muller, 1958): element
  ``2p`` is ``r cos(2 pi u2)`` and element ``2p + 1`` is ``r sin(2 pi u2)`` with
  ``r = sqrt(-2 ln u1)``, where ``u1`` and ``u2`` are draws ``2p`` and ``2p + 1``.
* Values are produced in float64 and rounded once (round-to-nearest-even) to the
  workload's dtype.

Seeds: ``1000 * workload_index + stream + 100 * b`` with streams Q=1, frame
latent=2, K noise=3, V=4, gates=5, compression weights=6, and ``b`` the batch
element.

The arithmetic runs in torch int64 / float64 on any device; int64 products wrap
modulo 2**64 and logical right shifts are written as arithmetic shift plus mask.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import torch

_GAMMA = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1
_CHUNK = 1 << 24  # elements per generation chunk (even)


def _i64(x: int) -> int:
    """Two's-complement int64 value with the same low 64 bits as ``x``."""
    x &= _MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    return (z >> k) & ((1 << (64 - k)) - 1)


def splitmix64_words(seed: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """Draws ``start .. start+count-1`` of SplitMix64 stream ``seed`` as int64 bit patterns."""
    c = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    z = c * _i64(_GAMMA) + _i64(seed)
    z = (z ^ _lsr(z, 30)) * _i64(_MIX1)
    z = (z ^ _lsr(z, 27)) * _i64(_MIX2)
    return z ^ _lsr(z, 31)


def splitmix64_reference(seed: int, count: int) -> List[int]:
    """Plain-Python SplitMix64 (arbitrary-precision ints), the definition itself."""
    out, state = [], seed & _MASK64
    for _ in range(count):
        state = (state + _GAMMA) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * _MIX1) & _MASK64
        z = ((z ^ (z >> 27)) * _MIX2) & _MASK64
        out.append(z ^ (z >> 31))
    return out


def uniform(seed: int, start: int, count: int, device="cpu") -> torch.Tensor:
    z = splitmix64_words(seed, start, count, device)
    return (_lsr(z, 11) + 1).to(torch.float64) * (2.0 ** -53)


def normal(seed: int, shape, device="cpu", dtype=torch.float64, scale: float = 1.0,
           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """N(0, scale^2) samples of stream ``seed`` laid out row-major in ``shape``."""
    n = int(math.prod(shape))
    if out is None:
        out = torch.empty(n, dtype=dtype, device=device)
    else:
        out = out.view(-1)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        lo = s - (s % 2)
        hi = e + (e % 2)
        npair = (hi - lo) // 2
        u = uniform(seed, lo, hi - lo, device).view(npair, 2)
        r = torch.sqrt(-2.0 * torch.log(u[:, 0]))
        th = (2.0 * math.pi) * u[:, 1]
        vals = torch.stack((r * torch.cos(th), r * torch.sin(th)), dim=1).view(-1)
        if scale != 1.0:
            vals = vals * scale
        out[s:e] = vals[s - lo: s - lo + (e - s)].to(out.dtype)
    return out.view(*shape)


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------
STREAM_Q, STREAM_LATENT, STREAM_KNOISE, STREAM_V, STREAM_GATES, STREAM_PHI = 1, 2, 3, 4, 5, 6
STREAM_LENS = 7
STREAM_HIDDEN, STREAM_WG, STREAM_BG = 8, 9, 10
HIDDEN = 3584  # hidden size of the Qwen2.5-VL-7B language model


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # seed base = 1000 * index
    dtype: str                 # "f32" | "bf16"
    batch: int
    kv_len: int
    q_len: int
    q_start: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    top_n: int
    window: int
    text_lead: int = 0         # text tokens before the video
    text_tail: int = 0         # text tokens after the video
    frame: int = 64            # video tokens per frame
    frame_corr: bool = False   # video K = frame latent + 0.5 * per-token noise
    gates: str = "sigmoid"     # "sigmoid" | "cmp" | "slc" | "swa"
    cmp_block: int = 32
    cmp_stride: int = 16
    sel_block: int = 64
    n_init: int = 1
    n_local: int = 2

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def params(self) -> Dict[str, float]:
        return dict(cmp_block=self.cmp_block, cmp_stride=self.cmp_stride, sel_block=self.sel_block,
                    top_n=self.top_n, n_init=self.n_init, n_local=self.n_local,
                    window=self.window, scale=0.0)

    def shape(self) -> Dict[str, int]:
        return dict(batch=self.batch, q_len=self.q_len, kv_len=self.kv_len, q_start=self.q_start,
                    num_q_heads=self.num_q_heads, num_kv_heads=self.num_kv_heads,
                    head_dim=self.head_dim)


def _prefill(name, index, dtype, T, Hq, Hkv, D, n, w, lead=0, tail=0, corr=False, gates="sigmoid"):
    return Workload(name=name, index=index, dtype=dtype, batch=1, kv_len=T, q_len=T, q_start=0,
                    num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, top_n=n, window=w,
                    text_lead=lead, text_tail=tail, frame_corr=corr, gates=gates)


# The five workloads of the layer: a tiny fp32 case, the Qwen2.5-VL-7B-shaped
# hybrid layer at 36K and 128K tokens (64 tokens per frame), a 16 x 64K decode
# step, and the 128K budget / gate sweep with 1 % text.
WORKLOADS: Dict[str, Workload] = {
    "tiny": _prefill("tiny-f32-T1024", 1, "f32", 1024, 4, 1, 64, 4, 128),
    "36k": _prefill("qwen2.5vl7b-36k", 2, "bf16", 36352, 28, 4, 128, 16, 512, 256, 256, True),
    "128k": _prefill("qwen2.5vl7b-128k", 3, "bf16", 131072, 28, 4, 128, 16, 512, 256, 256, True),
    "decode": Workload(name="decode-16x64k", index=4, dtype="bf16", batch=16, kv_len=65536, q_len=1,
                       q_start=65535, num_q_heads=28, num_kv_heads=4, head_dim=128, top_n=16,
                       window=512, frame_corr=True),
    "sweep": _prefill("sweep-128k-1pct-text", 5, "bf16", 131072, 28, 4, 128, 16, 512, 640, 640, True),
    # 16 sequences of mixed lengths (decode_lengths) in a paged cache of 64K-token capacity
    "decode_varlen": Workload(name="decode-varlen-paged-16x(4K..64K)", index=6, dtype="bf16", batch=16,
                              kv_len=65536, q_len=1, q_start=65535, num_q_heads=28, num_kv_heads=4,
                              head_dim=128, top_n=16, window=512, frame_corr=True),
}


def decode_lengths(wl: Workload, lo: int = 4096) -> List[int]:
    """Per-sequence token counts of a variable-length decode batch: seeded, uniform in [lo, kv_len]."""
    u = uniform(1000 * wl.index + STREAM_LENS, 0, wl.batch)
    return [int(lo + math.floor(x * (wl.kv_len - lo + 1))) for x in u.tolist()]

SWEEP_VARIANTS = [(n, w, g) for (n, w) in ((16, 512), (8, 256)) for g in ("sigmoid", "cmp", "slc")]

GATE_REGIMES = {"cmp": (0.9, 0.05, 0.05), "slc": (0.05, 0.9, 0.05), "swa": (0.05, 0.05, 0.9)}


def video_mask(wl: Workload, device="cpu") -> torch.Tensor:
    """is_video [B, q_len] (uint8) for the rows of Q (absolute positions q_start + r)."""
    pos = torch.arange(wl.q_start, wl.q_start + wl.q_len, device=device)
    vid = (pos >= wl.text_lead) & (pos < wl.kv_len - wl.text_tail)
    return vid.to(torch.uint8).unsqueeze(0).expand(wl.batch, wl.q_len).contiguous()


def make_inputs(wl: Workload, device="cpu", batch_offset: int = 0) -> Dict[str, torch.Tensor]:
    """All inputs of one workload, rounded to its dtype (gates and weights stay fp32).

    ``batch_offset`` shifts the batch index used in the seeds, so that several
    independent copies of a workload (e.g. rotating decode caches) can be drawn.
    """
    dt = wl.torch_dtype
    B, T, Tq, Hq, Hkv, D = wl.batch, wl.kv_len, wl.q_len, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    base = 1000 * wl.index
    q = torch.empty(B, Tq, Hq, D, dtype=dt, device=device)
    k = torch.empty(B, T, Hkv, D, dtype=dt, device=device)
    v = torch.empty(B, T, Hkv, D, dtype=dt, device=device)
    g = torch.empty(B, Tq, Hq, 3, dtype=torch.float32, device=device)
    n_video = T - wl.text_lead - wl.text_tail
    n_frames = (n_video + wl.frame - 1) // wl.frame
    for b in range(B):
        sb = base + 100 * (b + batch_offset)
        normal(sb + STREAM_Q, (Tq, Hq, D), device, out=q[b])
        normal(sb + STREAM_V, (T, Hkv, D), device, out=v[b])
        if wl.frame_corr and n_video > 0:
            kb = normal(sb + STREAM_KNOISE, (T, Hkv, D), device)
            lat = normal(sb + STREAM_LATENT, (n_frames, Hkv, D), device)
            vs, ve = wl.text_lead, T - wl.text_tail
            frame_of = (torch.arange(vs, ve, device=device) - vs) // wl.frame
            kb[vs:ve] = lat[frame_of] + 0.5 * kb[vs:ve]
            k[b].copy_(kb.to(dt))
            del kb, lat
        else:
            normal(sb + STREAM_KNOISE, (T, Hkv, D), device, out=k[b])
        if wl.gates == "sigmoid":
            x = normal(sb + STREAM_GATES, (Tq, Hq, 3), device)
            g[b] = (1.0 / (1.0 + torch.exp(-x))).to(torch.float32)
        else:
            g[b] = torch.tensor(GATE_REGIMES[wl.gates], dtype=torch.float32, device=device)
    w = normal(base + STREAM_PHI, (wl.cmp_block,), device, scale=1.0 / math.sqrt(wl.cmp_block))
    w = w.to(torch.float32)
    return dict(q=q, k=k, v=v, gates=g, w_k=w, w_v=w.clone(), is_video=video_mask(wl, device))


def make_gate_inputs(wl: Workload, device="cpu", hidden: int = HIDDEN, batch_offset: int = 0
                     ) -> Dict[str, torch.Tensor]:
    """Inputs of the gate projection for the query rows of a workload: hidden states x [B, q_len,
    hidden] ~ N(0, 1), weight w_g [3 Hq, hidden] ~ N(0, 1/hidden) (both rounded to the workload's
    dtype) and bias b_g [3 Hq] ~ N(0, 1/4) in fp32, so that the gate logits are about N(0, 1.25)."""
    dt = wl.torch_dtype
    B, Tq, N = wl.batch, wl.q_len, 3 * wl.num_q_heads
    base = 1000 * wl.index
    x = torch.empty(B, Tq, hidden, dtype=dt, device=device)
    for b in range(B):
        normal(base + 100 * (b + batch_offset) + STREAM_HIDDEN, (Tq, hidden), device, out=x[b])
    w = normal(base + STREAM_WG, (N, hidden), device, scale=1.0 / math.sqrt(hidden)).to(dt)
    bias = normal(base + STREAM_BG, (N,), device, scale=0.5).to(torch.float32)
    return dict(x=x, w_g=w, b_g=bias)


def small(wl: Workload, **kw) -> Workload:
    """A reduced copy of a workload (same structure), for parity tests."""
    return wl.with_(**kw)
