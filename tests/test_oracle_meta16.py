"""Pins of the oracle's binary16 metadata option: step D and zero z rounded
to binary16 (nearest, ties to even) and codes taken against the rounded
grid.

- the rounding against numpy's float32 -> float16 conversion (a library
  routine), on values across binades, exact ties, subnormals and the
  overflow threshold;
- the quantizer: stored D and z are binary16 values equal to the rounded
  fp32 step and minimum; the codes equal a brute-force numpy float32
  evaluation of clamp(rint((x - z) / D)) against that grid; every value
  inside the grid's span is within D/2 of its dequantised value, and values
  outside it map to the nearest end;
- with fp32 metadata the quantizer is unchanged (same codes, step, zero as
  the default call).
"""
import numpy as np
import pytest


def test_rounding_matches_numpy(orc):
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 5, 20000)).astype(np.float32)
    x = x[np.abs(x) < 65504]
    got = np.array([orc.round_fp16(v) for v in x], np.float32)
    assert np.array_equal(got, x.astype(np.float16).astype(np.float32))


def test_rounding_ties_subnormals_overflow(orc):
    cases = []
    for e in (-24, -20, -15, -14, -3, 0, 5, 14, 15):  # spacing 2^(e-10) in binade e (subnormal below -14)
        u = 2.0 ** max(e - 10, -24)
        for k in (1024, 1025, 1500, 2047):
            base = k * u if e >= -14 else (k % 1024) * u
            for f in (0.0, 0.25, 0.5, 0.75):  # exact ties at 0.5: even wins
                cases.append(np.float32(base + f * u))
    cases += [np.float32(v) for v in (65504.0, 65519.0, 2.0 ** -25, 2.0 ** -26, 3 * 2.0 ** -26, 1e-9)]
    for v in cases:
        for s in (1, -1):
            x = np.float32(s * v)
            want = np.float32(np.float16(x))
            assert orc.round_fp16(x) == want, (x, orc.round_fp16(x), want)
    assert orc.round_fp16(np.float32(65520.0)) == np.inf
    assert orc.round_fp16(np.float32(-70000.0)) == -np.inf


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("group", [32, 64])
def test_quantizer_with_binary16_metadata(orc, bits, group):
    rng = np.random.default_rng(bits * 100 + group)
    d, rows = 128, 300
    x = (rng.standard_normal((rows, d)) * rng.choice([1e-3, 0.3, 7.0, 900.0], size=(rows, 1))).astype(np.float32)
    x[0] = 0.0                       # zero step
    x[1, :group] = 2.0 ** -20        # a constant group of a subnormal-scale value
    x[2, :group] = np.linspace(-1e-5, 1e-5, group, dtype=np.float32)  # step in the binary16 subnormals
    codes, step, zero = orc.quantize(x, bits, group, meta="f16")
    top = (1 << bits) - 1
    ng = d // group
    xg = x.reshape(rows, ng, group)
    mn = xg.min(axis=2) + np.float32(0.0)
    mx = xg.max(axis=2) + np.float32(0.0)
    step32 = (mx - mn) / np.float32(top)
    assert np.array_equal(step, step32.astype(np.float16).astype(np.float32))
    assert np.array_equal(zero, mn.astype(np.float16).astype(np.float32))
    c = orc.unpack(codes, d, bits).reshape(rows, ng, group).astype(np.int64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (xg - zero[..., None]) / step[..., None]  # float32 IEEE division
    want = np.where(step[..., None] > 0, np.clip(np.rint(t), 0, top), 0).astype(np.int64)
    assert np.array_equal(c, want)
    xh = zero[..., None].astype(np.float64) + step[..., None].astype(np.float64) * c
    lo = zero[..., None].astype(np.float64)
    hi = lo + top * step[..., None].astype(np.float64)
    inside = (xg >= lo) & (xg <= hi)
    err = np.abs(xg - xh)
    assert np.all(err[inside] <= step[..., None].repeat(group, 2)[inside] / 2 * (1 + 1e-6) + 1e-30)
    assert np.all(xh[xg < lo] == lo.repeat(group, 2)[xg < lo])
    assert np.all(xh[xg > hi] == hi.repeat(group, 2)[xg > hi])


def test_fp32_metadata_unchanged(orc):
    x = np.random.default_rng(3).standard_normal((50, 128)).astype(np.float32)
    a = orc.quantize(x, 2, 64)
    b = orc.quantize(x, 2, 64, meta="f32")
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
