"""Softmax range on every attention kernel: logits far from zero, and logits
that rise or fall steeply along the keys, against the oracle.

The throughput kernel starts each row's running max at 0 and moves it only
when the row's sum leaves a fixed band after a tile (down when a row's first
visible tiles sum to almost nothing, up when a probability would overflow);
the short-query and general kernels start from -inf.  These inputs force
both directions deterministically:

  offset20   every logit of a row carries a common offset of about -20
             (natural units): the first tile's sum is far below the band,
             the running max moves down once;
  offset150  the same at about -150: the move is larger than 128 in the
             exp2 domain, beyond the finite range of the rescale factor;
  ramp_up    logits rise by about 120 along the keys (cache first, then
             the current chunk): the max moves down on the first tile and
             up again many times;
  ramp_down  the reverse: the first tile holds the largest logits.

Construction (input structure only): every channel of every key (cached
and current) gets mu_i added, every query channel nu, so the logit of key i
moves by nu * mu_i * d * tau plus per-key noise; everything is rounded to
bf16 and both the GPU and the oracle see the same values.  Softmax is
invariant to a common offset ("量化鍵值偷走注意力…" (agents-report.net),
§為何校正有效: one softmax over both segments), so the outputs stay O(1)
and the usual bar applies.
"""
import numpy as np
import pytest

from bit_kv_cache_03_amd import workloads as W
from _problems import oracle_problem

pytestmark = pytest.mark.gpu


def _shifted(w, data, case):
    """The workload's inputs with the offset or ramp of `case` built in."""
    f = lambda x: x.astype(np.float32) if x.dtype == np.float32 else W.bf16_to_f32(x)
    n = w.Nc + w.Ncur
    sqd = np.sqrt(w.d)  # nu * mu * d * tau with tau = 1 / sqrt(d)
    if case.startswith("offset"):
        target = float(case[len("offset"):])
        nu = np.sqrt(target / sqd)
        mu = np.full(n, nu, np.float32)
        nu = -nu
    else:
        nu = 2.0
        mu = np.linspace(-60.0, 60.0, n, dtype=np.float32) / (nu * sqd)
        if case == "ramp_down":
            mu = mu[::-1].copy()
    out = dict(data)
    out["q"] = W.bf16_bits(f(data["q"]) + np.float32(nu))
    out["kc"] = W.bf16_bits(f(data["kc"]) + mu[None, None, : w.Nc, None])
    out["k"] = W.bf16_bits(f(data["k"]) + mu[None, None, w.Nc:, None])
    for name in ("vc", "v"):
        out[name] = W.bf16_bits(f(data[name]))
    return out


RANGE_CASES = ["offset20", "offset150", "ramp_up", "ramp_down"]

# (kernel, workload, correction, path): the throughput kernel (d = 128, more
# than 64 rows per KV head, off / Taylor), the short-query kernel (d = 128,
# few rows), and the general kernel (the exact form at d = 128; d = 64)
KERNELS = {
    "throughput": (W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=1, Hq=2, Hkv=1, Nq=100, Ncur=100, Nc=700),
                   ("off", "taylor"), "long"),
    "short": (W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=1, Hq=4, Hkv=1, Nq=8, Ncur=40, Nc=900),
              ("off", "taylor"), "short"),
    "general_exact": (W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=1, Hkv=1, Nq=80, Ncur=80, Nc=500),
                      ("exact",), "long"),
    "general_exact_short": (W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=1, Hkv=1, Nq=16, Ncur=30, Nc=600),
                            ("exact",), "short"),
    "general_d64": (W.WORKLOADS["tiny_d64_int2"].scaled(Hq=2, Hkv=1, Nq=90, Ncur=90, Nc=520),
                    ("off", "taylor"), "long"),
}


def _run(orc, kernel, case, splits=0, causal=False):
    import _gpu
    w, corrs, path = KERNELS[kernel]
    data = _shifted(w, W.generate(w), case)
    kc = _gpu.build_cache(w, data["kc"], w.kbits)
    vc = _gpu.build_cache(w, data["vc"], w.vbits)
    for corr in corrs:
        print(f"[range] {case} kernel={kernel} d={w.d} Nq={w.Nq} Ncur={w.Ncur} Nc={w.Nc} corr={corr} "
              f"path={path} splits={splits} causal={causal}", flush=True)
        out = _gpu.run_attention(w, data, kc, vc, corr=corr, path=path, splits=splits, causal=causal)
        got = _gpu.out_rows(out)
        ref = oracle_problem(orc, w, corr, data=data, causal=causal).attention()
        _gpu.check(got, ref)


@pytest.mark.parametrize("case", RANGE_CASES)
@pytest.mark.parametrize("kernel", sorted(KERNELS))
def test_range(orc, kernel, case):
    _run(orc, kernel, case)


@pytest.mark.parametrize("case", RANGE_CASES)
@pytest.mark.parametrize("kernel", ["throughput", "short", "general_exact_short"])
def test_range_split(orc, kernel, case):
    """Forced key-range splits: every split starts its own running max, and
    the combine merges splits whose maxima lie far apart (ramps) or far
    below zero (offsets)."""
    _run(orc, kernel, case, splits=3)


@pytest.mark.parametrize("case", ["offset150", "ramp_up"])
@pytest.mark.parametrize("kernel", ["throughput", "short"])
def test_range_causal(orc, kernel, case):
    _run(orc, kernel, case, causal=True)
