"""Pins of the oracle's bfloat16 metadata option: step D and zero z rounded
to bfloat16 (nearest, ties to even) and codes taken against the rounded
grid.

- the rounding against torch's float32 -> bfloat16 conversion (a library
  routine), on values across binades, exact ties, fp32 and bfloat16
  subnormals and the overflow threshold; and, independently of any library,
  that the result is a bfloat16 value (low 16 bits zero) within half a
  spacing of x, with exact ties going to the even neighbour;
- the quantizer, groups along the head dimension and along the tokens:
  stored D and z are the bfloat16 roundings of the fp32 step and minimum;
  the codes equal a brute-force numpy float32 evaluation of
  clamp(rint((x - z) / D)) against that grid; every value inside the grid's
  span is within D/2 of its dequantised value and values outside it map to
  the nearest end.
"""
import numpy as np
import pytest
import torch


def _torch_bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def test_rounding_matches_torch(orc):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-37, 37, 20000)).astype(np.float32)
    got = np.array([orc.round_bf16(v) for v in x], np.float32)
    assert np.array_equal(got, _torch_bf16(x))


def test_rounding_ties_subnormals_overflow(orc):
    cases = []
    for e in (-149, -140, -133, -127, -126, -100, -3, 0, 5, 100, 127):  # binade [2^e, 2^(e+1))
        u = 2.0 ** max(e - 7, -133)  # bfloat16 spacing there
        for k in (128, 129, 200, 255):
            base = k * u if e >= -126 else (k % 128) * u
            for f in (0.0, 0.25, 0.5, 0.75, 0.5 + 2.0 ** -10):  # exact ties at 0.5: even wins
                v = np.float32(base + f * u)
                if v != 0 and np.isfinite(v):
                    cases.append(v)
    cases += [np.float32(v) for v in (2.0 ** -149, 3 * 2.0 ** -149, 2.0 ** -134, 3 * 2.0 ** -134, 1e-45)]
    for v in cases:
        for s in (1, -1):
            x = np.float32(s * v)
            r = np.float32(orc.round_bf16(x))
            assert r == _torch_bf16(x)[()], (x, r)
            # library-free checks: a bfloat16 value, nearest, ties to even
            if np.isinf(r):  # overflow: only from the upper half of the last spacing on
                assert abs(float(x)) >= (2 - 2.0 ** -8) * 2.0 ** 127, (x, r)
                continue
            rb = int(r.view(np.uint32))
            assert rb & 0xFFFF == 0, (x, r)
            u = 2.0 ** max(int(np.floor(np.log2(abs(float(x))))) - 7, -133)
            err = abs(float(r) - float(x))
            assert err <= u / 2, (x, r)
            if err == u / 2:
                assert (rb >> 16) & 1 == 0, (x, r)
    big = float(np.finfo(np.float32).max)
    assert orc.round_bf16(np.float32(big)) == np.inf  # past (2 - 2^-8) 2^127
    assert orc.round_bf16(np.float32((2 - 2.0 ** -7) * 2.0 ** 127)) == np.float32((2 - 2.0 ** -7) * 2.0 ** 127)
    assert orc.round_bf16(np.float32(-(2 - 2.0 ** -9) * 2.0 ** 127)) == -np.inf


def _check_grid(xg, step, zero, c, top):
    """xg: [..., group] values; step, zero: [...] stored bfloat16 values;
    c: [..., group] codes."""
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (xg - zero[..., None]) / step[..., None]  # float32 IEEE division
    want = np.where(step[..., None] > 0, np.clip(np.rint(t), 0, top), 0).astype(np.int64)
    assert np.array_equal(c, want)
    xh = zero[..., None].astype(np.float64) + step[..., None].astype(np.float64) * c
    lo = np.broadcast_to(zero[..., None].astype(np.float64), xg.shape)
    hi = lo + top * step[..., None].astype(np.float64)
    inside = (xg >= lo) & (xg <= hi)
    err = np.abs(xg - xh)
    half = np.broadcast_to(step[..., None], xg.shape) / 2
    assert np.all(err[inside] <= half[inside] * (1 + 1e-6) + 1e-45)
    assert np.all(xh[xg < lo] == lo[xg < lo])
    assert np.all(xh[xg > hi] == hi[xg > hi])


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("group", [32, 64, 128])
def test_quantizer_with_bfloat16_metadata(orc, bits, group):
    rng = np.random.default_rng(bits * 1000 + group)
    d, rows = 128, 300
    x = (rng.standard_normal((rows, d)) * rng.choice([1e-30, 1e-3, 0.3, 7.0, 900.0, 1e30], size=(rows, 1)))
    x = x.astype(np.float32)
    x[0] = 0.0                        # zero step
    x[1, :group] = 2.0 ** -130        # a constant group of an fp32-subnormal value
    x[2, :group] = np.linspace(-1e-38, 1e-38, group, dtype=np.float32)  # step in the bfloat16 subnormals
    x[3, :group] = 100.0 + np.linspace(0, 0.5, group, dtype=np.float32)  # |z| >> D: z's rounding moves the grid
    codes, step, zero = orc.quantize(x, bits, group, meta="bf16")
    top = (1 << bits) - 1
    ng = d // group
    xg = x.reshape(rows, ng, group)
    mn = xg.min(axis=2) + np.float32(0.0)
    mx = xg.max(axis=2) + np.float32(0.0)
    step32 = (mx - mn) / np.float32(top)
    assert np.array_equal(step, _torch_bf16(step32))
    assert np.array_equal(zero, _torch_bf16(mn))
    assert np.all(step.view(np.uint32) & 0xFFFF == 0) and np.all(zero.view(np.uint32) & 0xFFFF == 0)
    c = orc.unpack(codes, d, bits).reshape(rows, ng, group).astype(np.int64)
    _check_grid(xg, step, zero, c, top)


@pytest.mark.parametrize("bits", [2, 4])
def test_token_groups_with_bfloat16_metadata(orc, bits):
    """Groups of 64 consecutive tokens per channel (the last one shorter)."""
    rng = np.random.default_rng(40 + bits)
    B, H, N, d, G = 2, 3, 150, 128, 64
    x = (rng.standard_normal((B, H, N, d)) * rng.choice([0.01, 1.0, 50.0], size=(1, 1, 1, d))).astype(np.float32)
    codes, step, zero = orc.quantize(x, bits, G, meta="bf16", axis="tokens")
    top = (1 << bits) - 1
    c = orc.unpack(codes, d, bits).astype(np.int64)  # [B, H, N, d]
    for j in range(step.shape[2]):
        t0, t1 = j * G, min(N, (j + 1) * G)
        xg = np.moveaxis(x[:, :, t0:t1], 2, 3)       # [B, H, d, n]
        mn = xg.min(axis=3) + np.float32(0.0)
        mx = xg.max(axis=3) + np.float32(0.0)
        assert np.array_equal(step[:, :, j], _torch_bf16((mx - mn) / np.float32(top)))
        assert np.array_equal(zero[:, :, j], _torch_bf16(mn))
        _check_grid(xg, step[:, :, j], zero[:, :, j], np.moveaxis(c[:, :, t0:t1], 2, 3), top)


def test_bfloat16_differs_from_fp32_and_binary16(orc):
    """The three storage options give three different grids on data whose
    steps are not representable in 8 or 11 significant bits."""
    x = np.random.default_rng(7).standard_normal((64, 128)).astype(np.float32) * 3.1
    s32, sf16, sbf = (orc.quantize(x, 4, 64, meta=m)[1] for m in ("f32", "f16", "bf16"))
    assert not np.array_equal(s32, sbf) and not np.array_equal(sf16, sbf)
