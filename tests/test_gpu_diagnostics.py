"""kv_attention_diagnostics on the GPU against the oracle's kvo_diagnostics,
row by row, on seeded inputs with each workload's structure (several row
and key tiles, ragged tails, GQA, the causal mask, d = 64 and 128, INT2 and
INT4, all three correction modes).

Bars: the kernel's scores carry fp32 rounding (exact bf16 products for the
reference keys; the quantised keys as a bf16 hi + lo pair, ~2^-16 relative),
so log-sum-exps agree to 1e-3 + 1e-5 |lse|, masses to 2e-4 and KL to
2e-4 + 1e-3 KL.  Top-5 lists are compared by what is unique: at every rank
the oracle's score of the GPU's key equals the oracle's score at that rank
within the score error bound (near-ties may order either way), the lists
hold distinct visible keys, and they are equally long."""
import math

import numpy as np
import pytest

from bit_kv_cache_03_amd import workloads as W
from _problems import as_bf16, oracle_problem

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": (W.WORKLOADS["tiny_d64_int2"], False),
    "int4": (W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=2, Hkv=2, Nq=150, Ncur=150, Nc=333), False),
    "outliers": (W.WORKLOADS["h40_int2_outliers_cache25k"].scaled(Hq=2, Hkv=2, Nq=130, Ncur=130, Nc=300), False),
    "gqa_causal": (W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=2, Hq=8, Hkv=2, Nq=40, Ncur=50, Nc=333), True),
    "longvideo_causal": (W.WORKLOADS["long_video_cache61k"].scaled(Hq=1, Hkv=1, Nq=140, Ncur=100, Nc=400), True),
    "d64_group32": (W.WORKLOADS["tiny_d64_int2"].scaled(Hq=4, Hkv=2, Nq=70, Ncur=40, Nc=130, group=32, kbits=4), False),
    "no_cache": (W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=1, Hkv=1, Nq=70, Ncur=90, Nc=0), True),
}


def _scores(orc, w, data, corr, causal, row, meta="f32", kaxis="dim"):
    """Oracle scores of one row: quantised (kvo_logits) and reference."""
    p = oracle_problem(orc, w, corr, data=data, causal=causal, meta=meta, kaxis=kaxis)
    sq = p.logits(row)
    rep = w.Hq // w.Hkv
    b, h, j = row // (w.Hq * w.Nq), (row // w.Nq) % w.Hq, row % w.Nq
    q = W.bf16_to_f32(as_bf16(data["q"]))[b, h, j].astype(np.float64)
    keys = [W.bf16_to_f32(as_bf16(data[n]))[b, h // rep].astype(np.float64) for n in ("kc", "k")]
    keys = np.concatenate([k for k in keys if k.shape[0] > 0], axis=0)
    sr = (keys @ q) / math.sqrt(w.d)
    sr[~np.isfinite(sq)] = -np.inf
    return sr, sq


def check_top(got, want, s, label):
    """got/want: 5 key indices (-1 padded); s: the oracle's scores."""
    nv = int((want >= 0).sum())
    assert int((got >= 0).sum()) == nv, (label, got, want)
    g = got[:nv]
    assert len(set(g.tolist())) == nv and np.all(np.isfinite(s[g])), (label, got)
    eps = 1e-4 * max(1.0, float(np.max(np.abs(s[want[:nv]]))))
    assert np.all(np.abs(s[g] - s[want[:nv]]) <= eps), (label, got, want, s[g], s[want[:nv]])


def _compare(orc, w, causal, corr, data=None, max_rows=400, meta="f32", kaxis="dim"):
    import _gpu
    data = W.generate(w) if data is None else data
    print(f"[diagnostics] B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} Nq={w.Nq} Ncur={w.Ncur} Nc={w.Nc} "
          f"bits={w.kbits} group={w.group} corr={corr} causal={causal} meta={meta} kaxis={kaxis}", flush=True)
    kc = _gpu.build_cache(w, data["kc"], w.kbits, meta=meta, axis=kaxis) if w.Nc > 0 else None
    stats, tops = _gpu.run_diagnostics(w, data, kc, corr=corr, causal=causal)
    n = stats.shape[0]
    rows = np.arange(n) if n <= max_rows else np.linspace(0, n - 1, max_rows).astype(np.int64)
    ref, rtop = oracle_problem(orc, w, corr, data=data, causal=causal, meta=meta, kaxis=kaxis).diagnostics(
        as_bf16(data["kc"]), rows=rows)
    got = stats[rows]
    lse_err = np.abs(got[:, :2] - ref[:, :2]) - 1e-5 * np.abs(ref[:, :2])
    assert lse_err.max() <= 1e-3, lse_err.max()
    assert np.abs(got[:, 2:4] - ref[:, 2:4]).max() <= 2e-4, np.abs(got[:, 2:4] - ref[:, 2:4]).max()
    kl_err = np.abs(got[:, 4] - ref[:, 4]) - 1e-3 * np.abs(ref[:, 4])
    assert kl_err.max() <= 2e-4, kl_err.max()
    for i, row in enumerate(rows[:64]):
        sr, sq = _scores(orc, w, data, corr, causal, int(row), meta, kaxis)
        check_top(tops[row, 0], rtop[i, 0], sr, f"row {row} ref")
        check_top(tops[row, 1], rtop[i, 1], sq, f"row {row} q")
    return stats, ref


@pytest.mark.parametrize("corr", ["off", "taylor", "exact"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_diagnostics_parity(orc, case, corr):
    w, causal = CASES[case]
    _compare(orc, w, causal, corr)


def test_correction_restores_the_current_chunk_mass(orc):
    """The pages' claim measured through the GPU path: on INT2 keys with
    outlier channels the uncorrected cache takes attention from the current
    chunk, the Taylor correction gives most of it back."""
    import _gpu
    w = CASES["outliers"][0]
    data = W.generate(w)
    kc = _gpu.build_cache(w, data["kc"], w.kbits)
    off = _gpu.run_diagnostics(w, data, kc, corr="off")[0]
    tay = _gpu.run_diagnostics(w, data, kc, corr="taylor")[0]
    ref = off[:, 2].mean()
    assert off[:, 3].mean() < 0.5 * ref
    assert abs(tay[:, 3].mean() - ref) < 0.25 * abs(off[:, 3].mean() - ref)
    assert tay[:, 4].mean() < off[:, 4].mean()
