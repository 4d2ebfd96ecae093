"""Pins of the oracle's attention-balance statistics (kvo_diagnostics):
per query row, the softmax over the unquantised cached keys against the one
over the quantised (and corrected) cache.

- library routines: the same statistics from the oracle's own pinned logits
  (kvo_logits) and a numpy reference score matrix, through scipy's
  logsumexp, scipy.stats.entropy (KL divergence) and a stable lexsort for
  the top-5 (ties to the lower index), on shapes with many exact ties;
- special cases: a cache that quantises exactly gives identical statistics
  with the correction off; zero queries give uniform softmaxes (closed
  forms); rows with fewer than five visible keys pad the lists with -1;
- the pages' claim on synthetic data: quantisation without correction
  lowers the current chunk's mass, the Taylor correction restores most of
  it ("量化鍵值偷走注意力…" (agents-report.net), §問題 and §為何校正有效).
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp
from scipy.stats import entropy

from bit_kv_cache_03_amd import workloads as W
from _problems import as_bf16, oracle_problem


def _reference(orc, w, data, corr, causal, rows=None):
    """lse_ref, lse_q, mass_ref, mass_q, kl and both top-5 lists from
    library routines over the pinned quantised logits and numpy scores."""
    p = oracle_problem(orc, w, corr, data=data, causal=causal)
    tau = 1 / math.sqrt(w.d)
    q = W.bf16_to_f32(as_bf16(data["q"])).astype(np.float64)
    kref = W.bf16_to_f32(as_bf16(data["kc"])).astype(np.float64)
    kcur = W.bf16_to_f32(as_bf16(data["k"])).astype(np.float64)
    rep = w.Hq // w.Hkv
    n = w.Nc + w.Ncur
    rows = range(p.rows_total()) if rows is None else rows
    out, tops = [], []
    for row in rows:
        b, h, j = row // (w.Hq * w.Nq), (row // w.Nq) % w.Hq, row % w.Nq
        sq = p.logits(row)
        keys = np.concatenate([kref[b, h // rep], kcur[b, h // rep]], axis=0)
        sr = tau * (keys @ q[b, h, j])
        sr[~np.isfinite(sq)] = -np.inf  # the same mask
        vis = np.isfinite(sq)
        lr, lq = logsumexp(sr[vis]), logsumexp(sq[vis])
        pr, pq = np.exp(sr[vis] - lr), np.exp(sq[vis] - lq)
        cur = np.arange(n)[vis] >= w.Nc
        kl = entropy(pr, pq)
        out.append([lr, lq, pr[cur].sum(), pq[cur].sum(), kl])
        t = []
        for s in (sr, sq):
            order = np.lexsort((np.arange(n), -s))  # descending score, then lower index
            order = [int(i) for i in order if np.isfinite(s[i])][:5]
            t.append(order + [-1] * (5 - len(order)))
        tops.append(t)
    return np.array(out), np.array(tops)


def _tied(w, seed=3):
    """The workload's inputs moved onto coarse grids: many exact score ties."""
    data = W.generate(w)
    rng = np.random.default_rng(seed)
    f = lambda shape, lv: W.bf16_bits(rng.integers(-lv, lv + 1, size=shape).astype(np.float32) * 0.5)
    return dict(data, q=f(data["q"].shape, 1), kc=f(data["kc"].shape, 2), k=f(data["k"].shape, 2))


SHAPES = {
    "tiny": (W.WORKLOADS["tiny_d64_int2"].scaled(Nq=6, Ncur=9, Nc=40), False),
    "int4": (W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=2, Hkv=2, Nq=5, Ncur=7, Nc=70), False),
    "gqa_causal": (W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=1, Nq=6, Ncur=6, Nc=33), True),
    "outliers_causal": (W.WORKLOADS["h40_int2_outliers_cache25k"].scaled(Hq=1, Hkv=1, Nq=9, Ncur=5, Nc=50), True),
}


@pytest.mark.parametrize("tied", [False, True])
@pytest.mark.parametrize("corr", ["off", "taylor", "exact"])
@pytest.mark.parametrize("case", sorted(SHAPES))
def test_matches_library_statistics(orc, case, corr, tied):
    w, causal = SHAPES[case]
    data = _tied(w) if tied else W.generate(w)
    stats, top = oracle_problem(orc, w, corr, data=data, causal=causal).diagnostics(as_bf16(data["kc"]))
    ref, rtop = _reference(orc, w, data, corr, causal)
    assert np.allclose(stats, ref, rtol=1e-12, atol=1e-12), np.abs(stats - ref).max()
    assert np.array_equal(top, rtop)


def test_exact_cache_gives_identical_statistics(orc):
    """Keys on the INT2 grid {-1, -0.5, 0, 0.5} with both extremes in every
    group quantise exactly: with the correction off both softmaxes are the
    same (KL exactly 0, same lists, same masses)."""
    w = W.WORKLOADS["tiny_d64_int2"].scaled(Hq=2, Hkv=2, Nq=7, Ncur=11, Nc=60)
    data = W.generate(w)
    rng = np.random.default_rng(1)
    kc = rng.integers(0, 4, size=data["kc"].shape).astype(np.float32) * 0.5 - 1.0
    kc[..., ::w.group] = -1.0
    kc[..., 1::w.group] = 0.5
    data = dict(data, kc=kc)
    stats, top = oracle_problem(orc, w, "off", data=data).diagnostics(as_bf16(kc))
    assert np.array_equal(stats[:, 0], stats[:, 1])
    assert np.array_equal(stats[:, 2], stats[:, 3])
    assert np.all(stats[:, 4] == 0.0)
    assert np.array_equal(top[:, 0], top[:, 1])


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_are_uniform(orc, causal):
    w = W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=2, Hkv=1, Nq=4, Ncur=6, Nc=21)
    data = W.generate(w)
    data = dict(data, q=np.zeros_like(data["q"]))
    for corr in ("off", "taylor", "exact"):
        stats, top = oracle_problem(orc, w, corr, data=data, causal=causal).diagnostics(as_bf16(data["kc"]))
        for row in range(stats.shape[0]):
            j = row % w.Nq
            ncur = min(w.Ncur, j + w.Ncur - w.Nq + 1) if causal else w.Ncur
            n = w.Nc + ncur
            assert stats[row, 0] == pytest.approx(math.log(n), abs=1e-14)
            assert stats[row, 1] == pytest.approx(math.log(n), abs=1e-14)
            assert stats[row, 2] == pytest.approx(ncur / n, abs=1e-14)
            assert stats[row, 3] == pytest.approx(ncur / n, abs=1e-14)
            assert abs(stats[row, 4]) < 1e-14
            assert list(top[row, 0]) == list(range(5))  # all tied: the lowest indices


def test_rows_with_few_keys(orc):
    w = W.WORKLOADS["tiny_d64_int2"].scaled(Nq=3, Ncur=3, Nc=2)
    data = W.generate(w)
    stats, top = oracle_problem(orc, w, "taylor", data=data, causal=True).diagnostics(as_bf16(data["kc"]))
    for row in range(3):
        nvis = 2 + row + 1  # the cache and current keys 0..row
        for side in range(2):
            got = list(top[row, side])
            assert sorted(i for i in got if i >= 0) == sorted(set(i for i in got if i >= 0))
            assert sum(i >= 0 for i in got) == nvis and got[nvis:] == [-1] * (5 - nvis)
    assert np.all(stats[:, 4] >= 0)


def test_correction_restores_the_current_chunk_mass(orc):
    """The pages' claim: INT2 keys with outlier channels take attention from
    the current chunk when uncorrected; the Taylor correction gives most of
    it back, and moves the softmax closer to the unquantised one."""
    w = W.WORKLOADS["h40_int2_outliers_cache25k"].scaled(Hq=2, Hkv=2, Nq=32, Ncur=32, Nc=256)
    data = W.generate(w)
    res = {c: oracle_problem(orc, w, c, data=data).diagnostics(as_bf16(data["kc"]))[0] for c in ("off", "taylor")}
    ref = res["off"][:, 2].mean()
    off, tay = res["off"][:, 3].mean(), res["taylor"][:, 3].mean()
    assert off < 0.5 * ref
    assert abs(tay - ref) < 0.25 * abs(off - ref)
    assert res["taylor"][:, 4].mean() < res["off"][:, 4].mean()
