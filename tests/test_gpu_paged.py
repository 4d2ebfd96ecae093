"""The paged cache layout against the contiguous one, on the GPU: the same
tokens quantised through a shuffled page table (kv_quantize writing pool
rows) read back in logical order bit-exact, and every kernel path --
the throughput kernel (with and without the causal mask, split or not), the
short-query kernel, the general kernel (exact correction, d = 64) and the
diagnostics -- giving bit-identical results over both layouts (only the
addresses differ).  The contiguous results are pinned to the oracle by the
other parity tests."""
import numpy as np
import pytest
import torch

from bit_kv_cache_03_amd import kvq
from bit_kv_cache_03_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, page size, attention paths to run)
    "int4_long": (W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=2, Hkv=2, Nq=200, Ncur=200, Nc=333), 64),
    "gqa": (W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=3, Hq=8, Hkv=2, Nq=50, Ncur=50, Nc=700), 128),
    "outliers": (W.WORKLOADS["h40_int2_outliers_cache25k"].scaled(Hq=2, Hkv=2, Nq=150, Ncur=150, Nc=1000), 256),
    "d64": (W.WORKLOADS["tiny_d64_int2"].scaled(B=2, Hq=4, Hkv=2, Nq=77, Ncur=40, Nc=300, group=32, kbits=4), 64),
}


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))


@pytest.mark.parametrize("case", sorted(CASES))
def test_paged_matches_contiguous(case):
    import _gpu
    w, ps = CASES[case]
    print(f"[paged] {case} page_size={ps} B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Ncur={w.Ncur} Nc={w.Nc}",
          flush=True)
    data = W.generate(w)
    cap = (w.Nc + ps - 1) // ps * ps
    kc = _gpu.build_cache(w, data["kc"], w.kbits, cap=cap)
    vc = _gpu.build_cache(w, data["vc"], w.vbits, cap=cap)
    pk = _gpu.paged_cache(w, data["kc"], w.kbits, ps, cap=cap, seed=1)
    pv = _gpu.paged_cache(w, data["vc"], w.vbits, ps, cap=cap, seed=1)  # the same table contents
    assert torch.equal(pk.page_table, pv.page_table)
    pv.page_table = pk.page_table  # one table for K and V, as the attention call requires
    torch.cuda.synchronize()
    for c, p in ((kc, pk), (vc, pv)):
        for a, b in zip(c.logical(w.Nc), p.logical(w.Nc)):
            assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))
    print("    pools bit-exact in logical order", flush=True)
    runs = [("taylor", "long", 0, False), ("off", "long", 0, True), ("taylor", "short", 0, False),
            ("exact", "short", 0, False), ("exact", "long", 0, False), ("taylor", "long", 3, False),
            ("taylor", "short", 5, True)]
    for corr, path, splits, causal in runs:
        if causal and w.Nc == 0:
            continue
        a = _gpu.run_attention(w, data, kc, vc, corr=corr, path=path, splits=splits, causal=causal)
        b = _gpu.run_attention(w, data, pk, pv, corr=corr, path=path, splits=splits, causal=causal)
        assert _same(a, b), (corr, path, splits, causal)
    for corr in ("off", "taylor"):
        ra = _gpu.run_diagnostics(w, data, kc, corr=corr)
        rb = _gpu.run_diagnostics(w, data, pk, corr=corr)
        assert np.array_equal(ra[0], rb[0]) and np.array_equal(ra[1], rb[1]), corr
    print("    all paths identical", flush=True)


SMALL_PAGE_CASES = {
    # name: (workload, page size): pages that do not hold a whole 64-key tile
    "int4_p16": (W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=2, Hkv=2, Nq=150, Ncur=150, Nc=333), 16),
    "gqa_p32": (W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=2, Hq=8, Hkv=2, Nq=40, Ncur=40, Nc=500), 32),
    "gqa_p16": (W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=2, Hq=8, Hkv=2, Nq=3, Ncur=3, Nc=700), 16),
}


@pytest.mark.parametrize("case", sorted(SMALL_PAGE_CASES))
def test_small_pages(orc, case):
    """Pages of 16 and 32 tokens: the cache bit-exact in logical order, the
    attention (general kernel below 64 tokens per page, the short-query
    kernel from 32) against the oracle on both paths and all modes, and
    the diagnostics identical to the contiguous layout."""
    import _gpu
    from _problems import oracle_problem
    w, ps = SMALL_PAGE_CASES[case]
    print(f"[small pages] {case} page_size={ps} B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nc={w.Nc}", flush=True)
    data = W.generate(w)
    cap = (w.Nc + ps - 1) // ps * ps
    kc = _gpu.build_cache(w, data["kc"], w.kbits, cap=cap)
    pk = _gpu.paged_cache(w, data["kc"], w.kbits, ps, cap=cap, seed=7)
    pv = _gpu.paged_cache(w, data["vc"], w.vbits, ps, cap=cap, seed=7)
    pv.page_table = pk.page_table
    torch.cuda.synchronize()
    for a, b in zip(kc.logical(w.Nc), pk.logical(w.Nc)):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))
    for corr in ("off", "taylor", "exact"):
        ref = oracle_problem(orc, w, corr, data=data).attention()
        for path in ("long", "short"):
            got = _gpu.out_rows(_gpu.run_attention(w, data, pk, pv, corr=corr, path=path))
            _gpu.check(got, ref, label=f"{path} {corr} ")
    ra = _gpu.run_diagnostics(w, data, kc, corr="taylor")
    rb = _gpu.run_diagnostics(w, data, pk, corr="taylor")
    assert np.array_equal(ra[0], rb[0]) and np.array_equal(ra[1], rb[1])
