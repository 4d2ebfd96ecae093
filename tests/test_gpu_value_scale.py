"""Values scaled by 2^k, with k = 20 (far beyond the fp16 range) and
k = -20 (deep in its subnormals), on every attention path.

The kernels multiply values into the fp16 range before their PV products:
the throughput and general kernels by 2^-ev, with ev fixed per (b, KV head)
from a pre-pass bound on |v|; the short-query kernel by a per-block
exponent.  Quantising v 2^k gives the same codes with steps and zero
points times 2^k, and every scaling on the way is an exact power of two.
So the throughput and general kernels must return exactly 2^k times the
unscaled output, bit for bit, including their split partials and combines.
The short-query kernel folds its exponent into the exponential's argument,
which rounds differently once shifted by k, so it is held to the output
tolerance instead.  This pins the value exponents without the oracle; the
unscaled outputs are checked against the oracle elsewhere."""
import numpy as np
import pytest

from bit_kv_cache_03_amd import workloads as W

pytestmark = pytest.mark.gpu


def _scaled(x: np.ndarray, k: int) -> np.ndarray:
    """x times 2^k, exactly (bf16 bits or float32)."""
    if x.dtype == np.uint16:
        y = W.bf16_to_f32(x).astype(np.float32) * np.float32(2.0 ** k)
        out = W.bf16_bits(y)
        assert np.array_equal(W.bf16_to_f32(out), y)  # no rounding, no overflow
        return out
    return (x * np.float32(2.0 ** k)).astype(np.float32)


_H24 = W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=2, Hkv=2, Nq=200, Ncur=200, Nc=333)
_GQA = W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=2, Hq=8, Hkv=2, Nq=4, Ncur=4, Nc=700)
_D64 = W.WORKLOADS["tiny_d64_int2"].scaled(B=2, Hq=4, Hkv=2, Nq=77, Ncur=40, Nc=300, group=32)
_INT2 = W.WORKLOADS["long_video_cache61k"].scaled(B=2, Hq=1, Hkv=1, Nq=77, Ncur=0, Nc=63, group=128)

# label: (workload, corr, path, splits, axis, exact)
CASES = {
    "throughput": (_H24, "taylor", "long", 0, "dim", True),
    "throughput_split": (_H24, "taylor", "long", 3, "dim", True),
    "throughput_int2_short_cache": (_INT2, "off", "long", 0, "dim", True),
    "general_exact": (_H24, "exact", "long", 0, "dim", True),
    "general_d64": (_D64, "taylor", "long", 0, "dim", True),
    "general_short_split": (_GQA, "exact", "short", 4, "dim", True),
    "general_tokens": (_H24, "taylor", "long", 0, "tokens", True),
    "short": (_GQA, "taylor", "short", 0, "dim", False),
    "short_split": (_GQA, "off", "short", 5, "dim", False),
}


@pytest.mark.parametrize("k", [20, -20])
@pytest.mark.parametrize("case", sorted(CASES))
def test_values_scale_by_powers_of_two(case, k):
    import _gpu
    w, corr, path, splits, axis, exact = CASES[case]
    print(f"[value scale] {case} k={k} B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} Nq={w.Nq} Ncur={w.Ncur} Nc={w.Nc} "
          f"corr={corr} path={path} splits={splits} axis={axis}", flush=True)
    data = W.generate(w)
    kc = _gpu.build_cache(w, data["kc"], w.kbits, axis=axis)
    vc = _gpu.build_cache(w, data["vc"], w.vbits, axis=axis)
    base = _gpu.out_rows(_gpu.run_attention(w, data, kc, vc, corr=corr, path=path, splits=splits))

    sdata = dict(data)
    sdata["vc"] = _scaled(data["vc"], k)
    if w.Ncur > 0:
        sdata["v"] = _scaled(data["v"], k)
    svc = _gpu.build_cache(w, sdata["vc"], w.vbits, axis=axis)
    got = _gpu.out_rows(_gpu.run_attention(w, sdata, kc, svc, corr=corr, path=path, splits=splits))
    assert np.all(np.isfinite(got))
    want = base * 2.0 ** k
    if exact:
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (case, k, bad.size, got.flat[bad[0]], want.flat[bad[0]])
    else:
        _gpu.check(got * 2.0 ** -k, base, f"{case} k={k}")
