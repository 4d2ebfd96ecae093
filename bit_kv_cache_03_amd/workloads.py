"""Seeded synthetic workloads shaped like chunk-wise video-diffusion attention.

This module only draws random inputs; it holds none of the method's
arithmetic (no quantization, no attention, no correction).  Both the GPU tests
and the CPU oracle tests take their inputs from here, and so does the bench.

The Jensen-bias pages evaluate on video models (MAGI-1, SkyReels-V2,
HY-WorldPlay) and video benchmarks that are not available here; these
tensors stand in for them.  Chunk sizes are whole multiples of a 1560-token
frame (4680 = 3 frames, 6240 = 4) as in chunk-wise generation.

Recipe: ``numpy.random.default_rng([seed, stream])`` (PCG64) with
``seed = 20260525 + index`` of the workload; streams 0 q, 1 cached-K source,
2 cached-V source, 3 current K, 4 current V, 5 per-channel structure.  Values
are fp32 N(0,1) with the workload's structure applied, then rounded to bf16
(round to nearest even) except for the tiny fp32 workload.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np

BASE_SEED = 20260525


@dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed offset
    B: int
    Hq: int
    Hkv: int
    d: int
    Nq: int             # query rows per head (the current chunk)
    Ncur: int           # current-chunk keys/values (bf16)
    Nc: int             # cached tokens (quantized)
    kbits: int
    vbits: int
    group: int = 64
    src_dtype: str = "bf16"     # "bf16" or "f32" (the tiny workload)
    kstruct: str = "normal"     # "normal" | "outliers" | "loguniform"
    corr: str = "taylor"
    description: str = ""

    @property
    def rows_per_kvhead(self) -> int:
        return self.Nq * (self.Hq // self.Hkv)

    def scaled(self, **kw) -> "Workload":
        """Same structure, other sizes (for parity runs the oracle finishes)."""
        return replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("tiny_d64_int2", 0, B=1, Hq=1, Hkv=1, d=64, Nq=16, Ncur=16, Nc=256,
             kbits=2, vbits=2, src_dtype="f32",
             description="1x1 head, d=64, fp32 chunk of 16, 256 cached INT2 tokens"),
    Workload("h24_int4_cache16k", 1, B=1, Hq=24, Hkv=24, d=128, Nq=4096, Ncur=4096, Nc=16384,
             kbits=4, vbits=4,
             description="24 heads, d=128, chunk 4096, 16384 cached INT4/INT4 tokens"),
    Workload("h40_int2_outliers_cache25k", 2, B=1, Hq=40, Hkv=40, d=128, Nq=6240, Ncur=6240,
             Nc=24960, kbits=2, vbits=2, kstruct="outliers",
             description="40 heads, d=128, chunk 6240, 24960 cached INT2 tokens, "
                         "4 of 128 key channels x10"),
    Workload("gqa_prefill_b16_cache32k", 3, B=16, Hq=32, Hkv=8, d=128, Nq=512, Ncur=512,
             Nc=32768, kbits=2, vbits=4,
             description="batch 16, 32 query / 8 KV heads, chunk 512, 32768 cached "
                         "INT2-key / INT4-value tokens"),
    Workload("long_video_cache61k", 4, B=1, Hq=24, Hkv=24, d=128, Nq=4680, Ncur=4680,
             Nc=61440, kbits=2, vbits=2, kstruct="loguniform",
             description="24 heads, d=128, chunk 4680, 61440 cached INT2 tokens, "
                         "key channel std log-uniform in [0.5, 8]"),
]}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(w: Workload, stream: int, seed: Optional[int]) -> np.random.Generator:
    return np.random.default_rng([BASE_SEED + w.index if seed is None else seed, stream])


def _key_channel_scale(w: Workload, seed: Optional[int]) -> Optional[np.ndarray]:
    """Per (KV head, channel) multiplier applied to cached and current keys."""
    if w.kstruct == "normal":
        return None
    r = _rng(w, 5, seed)
    s = np.ones((w.Hkv, w.d), np.float32)
    if w.kstruct == "outliers":
        for h in range(w.Hkv):
            s[h, r.choice(w.d, size=4, replace=False)] = 10.0
    elif w.kstruct == "loguniform":
        s[:] = np.exp(r.uniform(np.log(0.5), np.log(8.0), size=(w.Hkv, w.d))).astype(np.float32)
    else:
        raise ValueError(w.kstruct)
    return s


def _normal(w: Workload, stream: int, shape, seed) -> np.ndarray:
    return _rng(w, stream, seed).standard_normal(size=shape, dtype=np.float32)


def generate(w: Workload, seed: Optional[int] = None, parts=("q", "kc", "vc", "k", "v")) -> Dict[str, np.ndarray]:
    """Draw the inputs of workload ``w``.

    Returns a dict with (as requested by ``parts``):
      q   [B][Hq][Nq][d]     queries
      k,v [B][Hkv][Ncur][d]  current-chunk keys / values
      kc,vc [B][Hkv][Nc][d]  cached-token keys / values before quantization
    as uint16 bf16 bits, or float32 for the fp32 workload.
    """
    ks = _key_channel_scale(w, seed)
    out = {}
    shapes = {"q": (w.B, w.Hq, w.Nq, w.d), "kc": (w.B, w.Hkv, w.Nc, w.d),
              "vc": (w.B, w.Hkv, w.Nc, w.d), "k": (w.B, w.Hkv, w.Ncur, w.d),
              "v": (w.B, w.Hkv, w.Ncur, w.d)}
    streams = {"q": 0, "kc": 1, "vc": 2, "k": 3, "v": 4}
    for name in parts:
        x = _normal(w, streams[name], shapes[name], seed)
        if ks is not None and name in ("kc", "k"):
            x *= ks[None, :, None, :]
        out[name] = x if w.src_dtype == "f32" else bf16_bits(x)
        del x
    return out


def cache_shapes(w: Workload, cap: Optional[int] = None):
    """Shapes of (codes, step, zero) of the K and V caches for capacity cap."""
    cap = w.Nc if cap is None else cap
    ng = w.d // w.group
    return ({"codes": (w.B, w.Hkv, cap, w.d * w.kbits // 8), "meta": (w.B, w.Hkv, cap, ng)},
            {"codes": (w.B, w.Hkv, cap, w.d * w.vbits // 8), "meta": (w.B, w.Hkv, cap, ng)})


def sample_rows(w: Workload, n: int, seed: int = 7) -> np.ndarray:
    """Flat query-row indices ((b*Hq + h)*Nq + j) for sampled parity checks:
    first and last rows of every head, the last (ragged) 64-row tile, and
    random rows."""
    total = w.B * w.Hq * w.Nq
    r = np.random.default_rng([BASE_SEED + w.index, 99, seed])
    picks = set()
    for bh in range(0, w.B * w.Hq, max(1, (w.B * w.Hq) // 8)):
        picks.update({bh * w.Nq, bh * w.Nq + w.Nq - 1})
    picks.update(range(max(0, total - 3), total))
    picks.update(r.choice(total, size=min(total, max(0, n - len(picks))), replace=False).tolist())
    return np.array(sorted(picks), dtype=np.int64)
