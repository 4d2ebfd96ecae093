"""Pins of the oracle's quantizer against things other than itself.

- hand-worked fixtures (tests/golden/quantizer_handworked.json);
- brute force: each code is the nearest grid point, ties to even, checked in
  exact rational arithmetic;
- the dequantization error bound |x - x^| <= step/2 (plus the rounding of
  step and of t);
- invariants: both extreme codes occur in every group with step > 0;
  scaling the input by 2^k scales step and zero exactly and keeps the codes;
  unpack(pack(c)) == c.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from bit_kv_cache_03_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantizer_handworked.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["id"])
def test_handworked_fixture(orc, case):
    x = np.array(case["x"], np.float32)[None, :]
    codes, step, zero = orc.quantize(x, case["bits"], case["group"])
    assert step[0].tolist() == case["step"]
    assert zero[0].tolist() == case["zero"]
    if "zero_sign_bit" in case:
        assert (zero[0].view(np.uint32) >> 31).tolist() == case["zero_sign_bit"]
    assert orc.unpack(codes, case["d"], case["bits"])[0].tolist() == case["codes"]
    if "packed_hex" in case:
        assert codes[0].tobytes().hex() == case["packed_hex"]
    # the bf16 entry point gives the same answer on bf16-exact inputs
    codes2, step2, zero2 = orc.quantize(W.bf16_bits(x), case["bits"], case["group"])
    assert np.array_equal(codes, codes2) and np.array_equal(step.view(np.uint32), step2.view(np.uint32))
    assert np.array_equal(zero.view(np.uint32), zero2.view(np.uint32))


def _near_tie(x, mn, step, c_lo):
    """True when the exact t lies within 2 fp32 ulps of a half-integer, where
    the fp32 rounding of t may legitimately move it across the tie."""
    t = (Fraction(float(x)) - Fraction(float(mn))) / Fraction(float(step))
    frac = t - int(t)
    ulp = Fraction(float(np.spacing(np.float32(max(float(t), 1.0)))))
    return abs(frac - Fraction(1, 2)) <= 2 * ulp


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_bruteforce_nearest_grid_point(orc, bits, src):
    rng = np.random.default_rng(11 + bits)
    rows, d, group = 48, 64, 32
    x = rng.standard_normal((rows, d)).astype(np.float32) * rng.choice([0.01, 1.0, 300.0], (rows, 1)).astype(np.float32)
    if src == "bf16":
        xb = W.bf16_bits(x)
        x = W.bf16_to_f32(xb)
        codes, step, zero = orc.quantize(xb, bits, group)
    else:
        codes, step, zero = orc.quantize(x, bits, group)
    c = orc.unpack(codes, d, bits)
    top = (1 << bits) - 1
    skipped = 0
    for r in range(rows):
        for g in range(d // group):
            seg = x[r, g * group:(g + 1) * group]
            mn, mx = float(seg.min()), float(seg.max())
            assert zero[r, g] == np.float32(mn)
            assert step[r, g] == np.float32(np.float32(mx) - np.float32(mn)) / np.float32(top)
            D = Fraction(float(step[r, g]))
            for k, v in enumerate(seg):
                # exact nearest grid point mn + j*D, j in [0, top], ties to even j
                best = None
                for j in range(top + 1):
                    dist = abs(Fraction(float(v)) - (Fraction(mn) + j * D))
                    if best is None or dist < best[0] or (dist == best[0] and j % 2 == 0):
                        best = (dist, j)
                got = int(c[r, g * group + k])
                if got != best[1]:
                    assert _near_tie(v, mn, step[r, g], best[1]), (r, g, k, float(v), got, best)
                    skipped += 1
    assert skipped <= rows * d // 200


@pytest.mark.parametrize("wname", sorted(W.WORKLOADS))
def test_error_bound_and_extreme_codes(orc, wname):
    w = W.WORKLOADS[wname]
    # a slice of the workload's own cache source (all heads, first 96 tokens)
    small = w.scaled(Nc=96, B=min(w.B, 2))
    src = W.generate(small, parts=("kc", "vc"))
    for name, bits in (("kc", w.kbits), ("vc", w.vbits)):
        xs = src[name]
        x = xs if xs.dtype == np.float32 else W.bf16_to_f32(xs)
        codes, step, zero = orc.quantize(xs, bits, w.group)
        xhat = orc.dequant(codes, step, zero, w.d, w.group, bits)
        st = np.repeat(step.astype(np.float64), w.group, axis=-1)
        mag = np.maximum(np.abs(np.repeat(zero, w.group, -1)), np.abs(x)).astype(np.float32)
        slack = 4 * np.spacing(mag).astype(np.float64)
        err = np.abs(x.astype(np.float64) - xhat)
        assert np.all(err <= st / 2 + slack), float((err - st / 2).max())
        c = orc.unpack(codes, w.d, bits).reshape(-1, w.d // w.group, w.group)
        has = step.reshape(-1, w.d // w.group) > 0
        assert np.all(c.min(-1)[has] == 0)
        assert np.all(c.max(-1)[has] == (1 << bits) - 1)


@pytest.mark.parametrize("k", [-3, 1, 5])
def test_power_of_two_scaling_is_exact(orc, k):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    for bits in (2, 4):
        c1, s1, z1 = orc.quantize(x, bits, 64)
        c2, s2, z2 = orc.quantize(x * np.float32(2.0 ** k), bits, 64)
        assert np.array_equal(c1, c2)
        assert np.array_equal(s1 * np.float32(2.0 ** k), s2)
        assert np.array_equal(z1 * np.float32(2.0 ** k), z2)


def test_pack_unpack_roundtrip(orc):
    rng = np.random.default_rng(3)
    for bits, d in ((2, 64), (2, 128), (4, 64), (4, 128)):
        c = rng.integers(0, 1 << bits, size=(17, d)).astype(np.uint8)
        p = orc.pack(c, bits)
        assert p.shape == (17, d * bits // 8)
        assert np.array_equal(orc.unpack(p, d, bits), c)


def test_adversarial_groups(orc):
    """Constant, two-valued, +-0, subnormal and large groups behave as the
    definition says (step 0 -> codes 0; two values -> extreme codes only)."""
    d = 64
    rows = []
    rows.append(np.full(d, 3.0, np.float32))                           # constant
    rows.append(np.where(np.arange(d) % 2 == 0, -1.0, 5.0).astype(np.float32))  # two-valued
    rows.append(np.where(np.arange(d) % 3 == 0, -0.0, 0.0).astype(np.float32))  # +-0 only
    tiny = np.float32(1e-45)
    rows.append((np.arange(d) % 4).astype(np.float32) * tiny)           # subnormals
    rows.append(np.linspace(0, 3.3895314e38, d).astype(np.float32))    # up to bf16 max
    x = np.stack(rows)
    codes, step, zero = orc.quantize(x, 2, 64)
    c = orc.unpack(codes, d, 2)
    assert step[0, 0] == 0 and np.all(c[0] == 0) and zero[0, 0] == 3.0
    assert step[1, 0] == np.float32(6.0) / np.float32(3.0)
    assert set(c[1].tolist()) == {0, 3}
    assert step[2, 0] == 0 and zero[2, 0].view(np.uint32) == 0 and np.all(c[2] == 0)
    assert np.all(np.isfinite(step)) and np.all(np.isfinite(zero))
    assert c[3].max() == 3 and c[3].min() == 0
    assert c[4, 0] == 0 and c[4, -1] == 3
