"""kv_attention_corrected on the GPU against the oracle, element by element.

Inputs are seeded and synthetic with each workload's structure, at sizes the
oracle finishes in seconds that still span several row tiles and key tiles
with ragged tails; both kernel paths, all three correction modes, and the
degenerate cases (no cache, no current chunk, one query row, head dim 64,
groups of 32/128, a non-default scale, GQA).  The oracle quantizes the
cache itself from the raw inputs; the GPU builds its own with kv_quantize.
Bar: max |out - ref| <= 2e-2 against the fp64 oracle and
mean |out - bf16(ref)| <= 1e-3 in the bf16 output format (see _gpu.check)."""
import numpy as np
import pytest
import torch

from bit_kv_cache_03_amd import workloads as W
from _problems import oracle_problem

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": W.WORKLOADS["tiny_d64_int2"],
    "int4": W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=2, Hkv=2, Nq=200, Ncur=200, Nc=333),
    "outliers": W.WORKLOADS["h40_int2_outliers_cache25k"].scaled(Hq=2, Hkv=2, Nq=150, Ncur=150, Nc=300),
    "gqa": W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=2, Hq=8, Hkv=2, Nq=50, Ncur=50, Nc=333),
    "longvideo": W.WORKLOADS["long_video_cache61k"].scaled(Hq=2, Hkv=2, Nq=130, Ncur=130, Nc=400),
}


def _compare(orc, w, corr, path, scale=0.0, splits=0, data=None, causal=False, meta="f32"):
    import _gpu
    data = W.generate(w) if data is None else data
    print(f"[attention] B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} Nq={w.Nq} Ncur={w.Ncur} Nc={w.Nc} "
          f"bits={w.kbits}/{w.vbits} group={w.group} corr={corr} path={path} splits={splits} causal={causal} "
          f"meta={meta}", flush=True)
    kc = _gpu.build_cache(w, data["kc"], w.kbits, meta=meta) if w.Nc > 0 else None
    vc = _gpu.build_cache(w, data["vc"], w.vbits, meta=meta) if w.Nc > 0 else None
    out = _gpu.run_attention(w, data, kc, vc, corr=corr, path=path, scale=scale, splits=splits, causal=causal)
    got = _gpu.out_rows(out)
    ref = oracle_problem(orc, w, corr, data=data, scale=scale, causal=causal, meta=meta).attention()
    _gpu.check(got, ref)
    return got, ref


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("corr", ["off", "taylor", "exact"])
@pytest.mark.parametrize("path", ["long", "short"])
def test_parity(orc, case, corr, path):
    _compare(orc, CASES[case], corr, path)


EDGE = {
    "no_cache": W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=2, Hkv=2, Nq=70, Ncur=90, Nc=0),
    "no_current": W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=2, Hkv=2, Nq=70, Ncur=0, Nc=150),
    "one_query": W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=1, Nq=1, Ncur=1, Nc=700),
    "one_key": W.WORKLOADS["h40_int2_outliers_cache25k"].scaled(Hq=1, Hkv=1, Nq=33, Ncur=0, Nc=1),
    # one cached key on the 16-row tiles: the output is that key's value, so
    # no averaging over keys hides the rounding of the value product
    "one_key_16rows": W.WORKLOADS["h40_int2_outliers_cache25k"].scaled(Hq=1, Hkv=1, Nq=16, Ncur=0, Nc=1),
    "one_key_gqa": W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=1, Nq=4, Ncur=0, Nc=1),
    "two_keys_int4": W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=2, Hkv=1, Nq=8, Ncur=1, Nc=1),
    "d64_group32": W.WORKLOADS["tiny_d64_int2"].scaled(Hq=4, Hkv=2, Nq=77, Ncur=40, Nc=130, group=32, kbits=4),
    "group32": W.WORKLOADS["h40_int2_outliers_cache25k"].scaled(Hq=2, Hkv=2, Nq=64, Ncur=64, Nc=200, group=32),
    "group128": W.WORKLOADS["long_video_cache61k"].scaled(Hq=2, Hkv=2, Nq=64, Ncur=64, Nc=200, group=128),
    "nq_ne_ncur": W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=3, Hkv=1, Nq=45, Ncur=111, Nc=129),
    "exact_tiles": W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=1, Hkv=1, Nq=128, Ncur=64, Nc=256),
}


@pytest.mark.parametrize("case", sorted(EDGE))
@pytest.mark.parametrize("path", ["long", "short"])
def test_edge_cases(orc, case, path):
    w = EDGE[case]
    if path == "short" and w.Nc == 0:
        pytest.skip("the split path needs cached tokens")
    for corr in ("off", "taylor", "exact"):
        _compare(orc, w, corr, path)


def test_explicit_scale(orc):
    _compare(orc, CASES["outliers"], "taylor", "long", scale=0.05)
    _compare(orc, CASES["gqa"], "exact", "short", scale=0.2)


@pytest.mark.parametrize("splits", [1, 3, 7, 64])
def test_split_counts(orc, splits):
    _compare(orc, CASES["gqa"], "taylor", "short", splits=splits)


@pytest.mark.parametrize("splits", [2, 3, 5, 100])
def test_long_path_split_counts(orc, splits):
    """Key-range splits of the throughput kernel, forced: 2 and 3 cut inside
    the cached segment, 5 also puts a boundary inside the current chunk, 100
    is clamped to one 64-key tile per split (ragged last tiles in both
    segments)."""
    _compare(orc, CASES["longvideo"], "taylor", "long", splits=splits)
    _compare(orc, CASES["gqa"], "off", "long", splits=splits)


def test_correction_matters_and_modes_differ(orc):
    """The GPU output moves with the correction the way the oracle's does."""
    w = CASES["outliers"]
    data = W.generate(w)
    outs = {c: _compare(orc, w, c, "long", data=data) for c in ("off", "taylor", "exact")}
    d_gpu = np.abs(outs["taylor"][0] - outs["off"][0]).mean()
    d_ref = np.abs(outs["taylor"][1] - outs["off"][1]).mean()
    assert d_ref > 1e-3 and abs(d_gpu - d_ref) < 0.1 * d_ref


def test_deterministic(orc):
    import _gpu
    w = CASES["gqa"]
    data = W.generate(w)
    kc = _gpu.build_cache(w, data["kc"], w.kbits)
    vc = _gpu.build_cache(w, data["vc"], w.vbits)
    for path in ("long", "short"):
        a = _gpu.run_attention(w, data, kc, vc, path=path)
        b = _gpu.run_attention(w, data, kc, vc, path=path)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _scaled(data, sq, sk, sv):
    """The workload's inputs with q, keys and values multiplied by powers of
    two (exact in bf16)."""
    f = {"q": sq, "kc": sk, "k": sk, "vc": sv, "v": sv}
    out = {}
    for name, x in data.items():
        x32 = (x.astype(np.uint32) << 16).view(np.float32) if x.dtype == np.uint16 else x
        out[name] = W.bf16_bits(x32 * np.float32(f[name]))
    return out


SCALES = {
    # tiny operands: logits x2^-14 (near-uniform attention), values x2^-10
    "small": (2.0 ** -6, 2.0 ** -8, 2.0 ** -10),
    # operands spread over ~20 binary orders with the logits unchanged: the
    # key/query exponent balance and the value exponents at range extremes
    "wide": (2.0 ** -6, 2.0 ** 6, 2.0 ** 10),
    # logits x4: sharply peaked rows
    "peaked": (2.0, 2.0, 1.0),
}


@pytest.mark.parametrize("scales", sorted(SCALES))
@pytest.mark.parametrize("path", ["long", "short"])
def test_scaled_inputs(orc, scales, path):
    """Inputs far from unit size.  Outputs are linear in the values, so both
    sides are divided by the value factor before the comparison, and the bar
    is the usual one for every scale."""
    import _gpu
    sq, sk, sv = SCALES[scales]
    for case in ("gqa", "longvideo"):
        w = CASES[case]
        data = _scaled(W.generate(w), sq, sk, sv)
        for corr in ("off", "taylor"):
            print(f"[scaled] {scales} q x{sq} k x{sk} v x{sv} {case} corr={corr} path={path}", flush=True)
            kc = _gpu.build_cache(w, data["kc"], w.kbits)
            vc = _gpu.build_cache(w, data["vc"], w.vbits)
            out = _gpu.run_attention(w, data, kc, vc, corr=corr, path=path)
            got = _gpu.out_rows(out)
            ref = oracle_problem(orc, w, corr, data=data).attention()
            _gpu.check(got / sv, ref / sv)


# Causal mask within the current chunk, aligned to its end (query j of Nq
# sees current keys i <= j + Ncur - Nq, and the whole cache).
CAUSAL = {
    "square": CASES["int4"],
    "gqa": CASES["gqa"],  # 4 query heads per KV head: row blocks span several heads
    "nq_lt_ncur": EDGE["nq_ne_ncur"],
    "nq_gt_ncur": W.WORKLOADS["h40_int2_outliers_cache25k"].scaled(Hq=2, Hkv=2, Nq=150, Ncur=70, Nc=300),
    "rows3": W.WORKLOADS["long_video_cache61k"].scaled(Hq=1, Hkv=1, Nq=600, Ncur=600, Nc=100),  # 3 row blocks
    "no_cache": W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=1, Hkv=1, Nq=300, Ncur=300, Nc=0),
    "d64": W.WORKLOADS["tiny_d64_int2"].scaled(Hq=4, Hkv=2, Nq=40, Ncur=77, Nc=130, group=32, kbits=4),
}


@pytest.mark.parametrize("case", sorted(CAUSAL))
@pytest.mark.parametrize("path", ["long", "short"])
def test_causal(orc, case, path):
    w = CAUSAL[case]
    if path == "short" and w.Nc == 0:
        pytest.skip("the split path needs cached tokens")
    data = W.generate(w)
    for corr in ("off", "taylor", "exact"):
        _compare(orc, w, corr, path, data=data, causal=True)


@pytest.mark.parametrize("splits", [2, 3, 7, 40])
@pytest.mark.parametrize("path", ["long", "short"])
def test_causal_split_counts(orc, splits, path):
    """Forced key-range splits under the mask: late splits hold only
    current keys, some of them hidden from every row of a workgroup or
    from some of its rows."""
    for case in ("rows3", "gqa"):
        _compare(orc, CAUSAL[case], "taylor", path, splits=splits, causal=True)


def test_causal_one_query_is_unmasked(orc):
    """With one query row (decode) the mask hides nothing."""
    import _gpu
    w = W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=2, Nq=1, Ncur=37, Nc=500)
    data = W.generate(w)
    kc = _gpu.build_cache(w, data["kc"], w.kbits)
    vc = _gpu.build_cache(w, data["vc"], w.vbits)
    for path in ("long", "short"):
        a = _gpu.run_attention(w, data, kc, vc, path=path)
        b = _gpu.run_attention(w, data, kc, vc, path=path, causal=True)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_long_path_tail_split(orc):
    """300 work units (one 100-row block per head) on 256 CUs: the library
    runs 256 units over all keys and splits the 44 others into 5 key ranges
    (the tail of the last round); rows of both kinds against the oracle."""
    import _gpu
    from bit_kv_cache_03_amd import kvq
    w = W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=300, Hkv=300, Nq=100, Ncur=100, Nc=500)
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the split plan under test assumes 256 CUs")
    data = W.generate(w)
    kc = _gpu.build_cache(w, data["kc"], w.kbits)
    vc = _gpu.build_cache(w, data["vc"], w.vbits)
    q = _gpu.as_bf16_dev(data["q"])
    args = kvq.make_args(q, _gpu.as_bf16_dev(data["k"]), _gpu.as_bf16_dev(data["v"]), kc, vc, w.Nc,
                         torch.empty_like(q), corr="taylor")
    partials = 5 * w.B * w.Hq * w.Nq * (w.d + 4) * 4
    assert kvq.workspace_size(args) == partials + 300 * 384  # 5 key ranges; bounds of 300 KV heads
    out = _gpu.run_attention(w, data, kc, vc, corr="taylor")
    heads = [0, 1, 128, 255, 256, 257, 280, 299]  # units 256.. are the split tail
    rows = np.array([h * w.Nq + j for h in heads for j in (0, 37, 99)], dtype=np.int64)
    got = _gpu.out_rows(out, rows)
    ref = oracle_problem(orc, w, "taylor", data=data).attention(rows=rows)
    _gpu.check(got, ref)
