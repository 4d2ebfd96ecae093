"""The caches' running bound, on the GPU.

kv_quantize and the fused append raise, per (b, head), the largest
max(|z|, |z + (2^bits - 1) D|) over the groups they write; the attention
pre-passes read it instead of scanning every step and zero point.  Checked:
the bound equals that maximum over the oracle quantizer's steps and zero
points (all layouts: head-dimension and token groups, binary16 metadata,
paged pools, appends in chunks); the fused append leaves the same bound as
kv_quantize; attention outputs are bit-identical with and without it on
the throughput and general kernels (the bound equals the scan it replaces);
the short kernels, which with the bound fix their power-of-two block scales
once instead of raising them block by block, meet the oracle's bar both ways.
"""
import numpy as np
import pytest
import torch

from bit_kv_cache_03_amd import kvq
from bit_kv_cache_03_amd import workloads as W

pytestmark = pytest.mark.gpu

H24, GQA = W.WORKLOADS["h24_int4_cache16k"], W.WORKLOADS["gqa_prefill_b16_cache32k"]
LV, TINY = W.WORKLOADS["long_video_cache61k"], W.WORKLOADS["tiny_d64_int2"]
OUT = W.WORKLOADS["h40_int2_outliers_cache25k"]


def _expected(orc, src, bits, w, meta, axis):
    """max over each (b, h)'s groups of max(|z|, |z + top D|), with the fp32 fma
    the kernels use (exact in fp64, rounded once)."""
    _, step, zero = orc.quantize(src, bits, w.group, meta=meta, axis=axis)  # the input the cache was built from
    top = float((1 << bits) - 1)
    hi = (zero.astype(np.float64) + top * step.astype(np.float64)).astype(np.float32)
    g = np.maximum(np.abs(zero.astype(np.float32)), np.abs(hi))
    return g.reshape(g.shape[0], g.shape[1], -1).max(axis=2)


CASES = {
    # name: (workload, meta, axis, page size, chunk)
    "int4_dim": (H24.scaled(B=2, Hq=3, Hkv=3, Nc=333, Ncur=97), "f32", "dim", 0, 97),
    "int2_loguniform_m16": (LV.scaled(Hq=4, Hkv=4, Nc=500, Ncur=128), "f16", "dim", 0, 128),
    "gqa_paged": (GQA.scaled(B=3, Hq=8, Hkv=2, Nc=640, Ncur=64), "f32", "dim", 64, 64),
    "tokens": (H24.scaled(Hq=2, Hkv=2, Nc=256, Ncur=64), "f32", "tokens", 0, 64),
    "d64": (TINY.scaled(B=2, Hq=2, Hkv=2, Nc=300, group=32), "f32", "dim", 0, 50),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_bound_after_quantize(orc, case):
    import _gpu
    w, meta, axis, ps, chunk = CASES[case]
    print(f"[bound] {case}: B={w.B} Hkv={w.Hkv} Nc={w.Nc} d={w.d} g{w.group} meta={meta} axis={axis} page={ps}",
          flush=True)
    data = W.generate(w, parts=("kc", "vc"))
    for name, bits in (("kc", w.kbits), ("vc", w.vbits)):
        c = (_gpu.paged_cache(w, data[name], bits, ps, chunk=chunk, meta=meta, axis=axis) if ps else
             _gpu.build_cache(w, data[name], bits, chunk=chunk, meta=meta, axis=axis))
        torch.cuda.synchronize()
        got = c.bound.cpu().numpy()
        want = _expected(orc, data[name], bits, w, meta, axis)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (name, got, want)


def _clone(c):
    d = kvq.QCache.__new__(kvq.QCache)
    d.__dict__.update(c.__dict__)
    d.codes, d.scale, d.zero = c.codes.clone(), c.scale.clone(), c.zero.clone()
    d.bound = None if c.bound is None else c.bound.clone()
    return d


def _without_bound(c):
    d = kvq.QCache.__new__(kvq.QCache)
    d.__dict__.update(c.__dict__)
    d.bound = None
    return d


RUNS = {
    # name: (workload, corr, path, splits, bit-identical): the throughput kernel
    # (key and value bounds from the cache), the general kernel (value bound),
    # the short kernels (block scales fixed from the bound, else raised per block)
    "fast": (H24.scaled(Hq=2, Hkv=2, Nq=200, Ncur=200, Nc=300), "taylor", "long", 0, True),
    "fast_split": (GQA.scaled(B=2, Hq=8, Hkv=2, Nq=100, Ncur=100, Nc=700), "off", "long", 3, True),
    "general_exact": (H24.scaled(Hq=2, Hkv=2, Nq=64, Ncur=64, Nc=150), "exact", "long", 0, True),
    "general_d64": (TINY.scaled(B=2, Hq=4, Hkv=2, Nq=40, Ncur=40, Nc=200, group=32), "taylor", "long", 0, True),
    "short16": (GQA.scaled(B=2, Hq=8, Hkv=2, Nq=2, Ncur=2, Nc=900), "taylor", "short", 0, False),
    "short16_loguniform": (LV.scaled(Hq=2, Hkv=1, Nq=4, Ncur=4, Nc=700), "taylor", "short", 3, False),
    "short32_outliers": (OUT.scaled(Hq=2, Hkv=2, Nq=24, Ncur=24, Nc=600), "taylor", "short", 0, False),
}


@pytest.mark.parametrize("case", sorted(RUNS))
def test_attention_with_and_without_bound(orc, case):
    """All written rows are attended to.  Where the kernel only uses the bound
    in place of its own scan the outputs are bit-identical; elsewhere both meet
    the oracle's bar."""
    import _gpu
    from _problems import oracle_problem
    w, corr, path, splits, same = RUNS[case]
    print(f"[bound] attention {case}: {corr} {path} splits={splits}", flush=True)
    data = W.generate(w)
    kc = _gpu.build_cache(w, data["kc"], w.kbits)
    vc = _gpu.build_cache(w, data["vc"], w.vbits)
    a = _gpu.run_attention(w, data, kc, vc, corr=corr, path=path, splits=splits)
    b = _gpu.run_attention(w, data, _without_bound(kc), _without_bound(vc), corr=corr, path=path, splits=splits)
    if same:
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        return
    ref = oracle_problem(orc, w, corr, data=data).attention()
    _gpu.check(_gpu.out_rows(a), ref, "with bound: ")
    _gpu.check(_gpu.out_rows(b), ref, "without:    ")


def test_fused_append_raises_bound():
    import _gpu
    w = GQA.scaled(B=2, Hq=8, Hkv=2, Nq=64, Ncur=64, Nc=256)
    data = W.generate(w)
    kc = _gpu.build_cache(w, data["kc"], w.kbits, cap=w.Nc + w.Ncur)
    vc = _gpu.build_cache(w, data["vc"], w.vbits, cap=w.Nc + w.Ncur)
    kc2, vc2 = _clone(kc), _clone(vc)
    q, k, v = (_gpu.as_bf16_dev(data[x]) for x in ("q", "k", "v"))
    kvq.attention(q, k, v, kc, vc, w.Nc, append=True)
    kvq.quantize(k, kc2, w.Nc)
    kvq.quantize(v, vc2, w.Nc)
    torch.cuda.synchronize()
    assert torch.equal(kc.bound, kc2.bound) and torch.equal(vc.bound, vc2.bound)
    assert bool((kc.bound > 0).all()) and bool((vc.bound > 0).all())
