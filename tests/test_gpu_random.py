"""Seeded random configurations against the oracle: every option of the
attention call drawn together (shape, GQA ratio, bits, group, correction
mode, path, key-range splits, causal mask, paged layout, 16-bit metadata,
groups along the tokens), at sizes the oracle finishes in well under a
second.  The list is fixed by its seed; each case prints its options before
it runs."""
import os

import numpy as np
import pytest

from bit_kv_cache_03_amd import workloads as W
from _problems import oracle_problem

pytestmark = pytest.mark.gpu

BASES = ["tiny_d64_int2", "h24_int4_cache16k", "h40_int2_outliers_cache25k", "gqa_prefill_b16_cache32k",
         "long_video_cache61k"]


def _cases(n=600, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        base = W.WORKLOADS[BASES[rng.integers(len(BASES))]]
        d = base.d
        hkv = int(rng.choice([1, 2, 3]))
        gq = int(rng.choice([1, 2, 4]))
        axis_k = "tokens" if rng.random() < 0.25 else "dim"
        axis_v = "tokens" if rng.random() < 0.2 else "dim"
        group = int(rng.choice([g for g in (32, 64, 128) if g <= d or "tokens" in (axis_k, axis_v)]))
        if group > d and (axis_k == "dim" or axis_v == "dim"):
            group = d
        nq = int(rng.choice([1, 3, 16, 40, 77, 130, 200]))
        ncur = int(rng.choice([0, 1, nq, nq + int(rng.integers(1, 90))]))
        nc = int(rng.choice([0, 1, 63, 64, 65, 200, 333, 700]))
        if nc + ncur == 0:
            nc = 100
        causal = bool(rng.random() < 0.3) and not (nc == 0 and nq > ncur)
        corr = str(rng.choice(["off", "taylor", "exact"]))
        path = str(rng.choice(["auto", "long", "short"]))
        if path == "short" and nc == 0:
            path = "auto"
        splits = int(rng.choice([0, 0, 2, 5]))
        paged = bool(rng.random() < 0.3) and nc > 0
        # pages of 16..128 tokens (token groups need whole groups per page)
        ps = max(int(rng.choice([16, 32, 64, 128])), group if "tokens" in (axis_k, axis_v) else 16) if paged else 0
        r = rng.random()  # one draw, as before bfloat16 took half of the 16-bit share
        meta = "f16" if r < 0.15 else "bf16" if r < 0.3 else "f32"
        w = base.scaled(B=int(rng.choice([1, 2])), Hq=hkv * gq, Hkv=hkv, Nq=nq, Ncur=ncur, Nc=nc, group=group,
                        kbits=int(rng.choice([2, 4])), vbits=int(rng.choice([2, 4])))
        out.append((i, w, corr, path, splits, causal, ps, meta, axis_k, axis_v))
    return out


# KVQ_RANDOM_SEEDS="1,2" (and KVQ_RANDOM_N, cases per seed) swaps in other
# lists; by default the one list above, 600 cases.
_SEEDS = [int(x) for x in os.environ.get("KVQ_RANDOM_SEEDS", "20261203").split(",") if x]
CASES = [c for sd in _SEEDS for c in _cases(int(os.environ.get("KVQ_RANDOM_N", "600")), sd)]


@pytest.mark.parametrize("case", CASES, ids=[f"r{c[0]}" if len(_SEEDS) == 1 else f"s{j // max(1, len(CASES) // len(_SEEDS))}r{c[0]}"
                                             for j, c in enumerate(CASES)])
def test_random_configuration(orc, case):
    import _gpu
    i, w, corr, path, splits, causal, ps, meta, axis_k, axis_v = case
    paged = ps > 0
    print(f"[random r{i}] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} Nq={w.Nq} Ncur={w.Ncur} Nc={w.Nc} "
          f"bits={w.kbits}/{w.vbits} group={w.group} corr={corr} path={path} splits={splits} causal={causal} "
          f"page_size={ps} meta={meta} axes={axis_k}/{axis_v}", flush=True)
    data = W.generate(w)
    kc = vc = None
    if w.Nc > 0:
        mult = 1
        if "tokens" in (axis_k, axis_v):
            mult = max(mult, w.group)
        cap = -(-w.Nc // mult) * mult
        if paged:
            cap = -(-cap // ps) * ps
            kc = _gpu.paged_cache(w, data["kc"], w.kbits, ps, cap=cap, seed=i, meta=meta, axis=axis_k)
            vc = _gpu.paged_cache(w, data["vc"], w.vbits, ps, cap=cap, seed=i, meta=meta, axis=axis_v)
            vc.page_table = kc.page_table
        else:
            kc = _gpu.build_cache(w, data["kc"], w.kbits, cap=cap, meta=meta, axis=axis_k)
            vc = _gpu.build_cache(w, data["vc"], w.vbits, cap=cap, meta=meta, axis=axis_v)
    out = _gpu.run_attention(w, data, kc, vc, corr=corr, path=path, splits=splits, causal=causal)
    got = _gpu.out_rows(out)
    ref = oracle_problem(orc, w, corr, data=data, causal=causal, meta=meta, kaxis=axis_k, vaxis=axis_v).attention()
    _gpu.check(got, ref)
