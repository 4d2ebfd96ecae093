"""Caches grouped along the tokens (per channel) on the short-query path: the
16-row kernel's token-axis instances (at most 16 query rows per KV head) and
the 32-row kernel's (more rows, fp32 metadata), on the GPU against the
oracle.

Keys along the tokens (KIVI-style, values along the head dimension): the
kernel folds each token group's steps into the query and feeds the raw
codes to the MFMA, adding q.z and the per-channel Taylor bias per row
("量化鍵值偷走注意力…" (agents-report.net) §方法: one step per group or per
channel).  Values along the tokens (with keys either way, fp32 metadata):
dequantised with per-channel operands staged per token group.  Cases: token
groups of 32/64/128, INT2 and INT4 keys and values, decode and GQA chunks
(1-16 rows), ragged and tiny caches (the last token group shorter, fewer
keys than a block, one key), forced split counts, the causal mask, binary16
and bfloat16 metadata, paged pools (bit-identical to contiguous), keys with
large per-channel offsets (outlier channels) and log-uniform scales.  Bar:
that of every attention parity test."""
import numpy as np
import pytest
import torch

from bit_kv_cache_03_amd import kvq
from bit_kv_cache_03_amd import workloads as W
from _problems import oracle_problem

pytestmark = pytest.mark.gpu

GQA, H24 = W.WORKLOADS["gqa_prefill_b16_cache32k"], W.WORKLOADS["h24_int4_cache16k"]
OUT, LV = W.WORKLOADS["h40_int2_outliers_cache25k"], W.WORKLOADS["long_video_cache61k"]

CASES = {
    # name: workload (rows per KV head = Nq * Hq / Hkv <= 16)
    "gqa_decode_g64": GQA.scaled(B=2, Hq=8, Hkv=2, Nq=1, Ncur=1, Nc=1000, group=64),
    "gqa_chunk4_g32": GQA.scaled(B=2, Hq=8, Hkv=2, Nq=4, Ncur=4, Nc=777, group=32),
    "gqa_g128_ragged": GQA.scaled(B=1, Hq=8, Hkv=2, Nq=3, Ncur=5, Nc=1100, group=128),
    "int4_rows16": H24.scaled(B=1, Hq=2, Hkv=2, Nq=16, Ncur=16, Nc=700, group=64),
    "int4_k2_v4": H24.scaled(B=1, Hq=4, Hkv=2, Nq=5, Ncur=7, Nc=650, group=64, kbits=2),
    "outliers_decode": OUT.scaled(Hq=4, Hkv=2, Nq=1, Ncur=1, Nc=900, group=64),
    "longvideo_decode": LV.scaled(Hq=2, Hkv=2, Nq=1, Ncur=1, Nc=1300, group=128),
    "small_cache": GQA.scaled(B=2, Hq=8, Hkv=2, Nq=2, Ncur=2, Nc=20, group=32),
    "one_key": GQA.scaled(B=1, Hq=8, Hkv=2, Nq=1, Ncur=0, Nc=1, group=64),
    "no_current": H24.scaled(B=1, Hq=2, Hkv=2, Nq=8, Ncur=0, Nc=513, group=32),
}


def _caches(w, data, meta="f32", page=0, seed=0, kaxis="tokens", vaxis="dim"):
    import _gpu
    cap = -(-w.Nc // w.group) * w.group
    if page:
        cap = -(-cap // page) * page
        kc = _gpu.paged_cache(w, data["kc"], w.kbits, page, cap=cap, seed=seed, meta=meta, axis=kaxis)
        vc = _gpu.paged_cache(w, data["vc"], w.vbits, page, cap=cap, seed=seed, meta=meta, axis=vaxis)
        vc.page_table = kc.page_table  # one table, as the attention call requires
        return kc, vc
    return (_gpu.build_cache(w, data["kc"], w.kbits, cap=cap, meta=meta, axis=kaxis),
            _gpu.build_cache(w, data["vc"], w.vbits, cap=cap, meta=meta, axis=vaxis))


def _compare(orc, w, corr, splits=0, causal=False, meta="f32", page=0, kaxis="tokens", vaxis="dim"):
    import _gpu
    data = W.generate(w)
    print(f"[tokens short] B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Ncur={w.Ncur} Nc={w.Nc} bits={w.kbits}/{w.vbits} "
          f"group={w.group} corr={corr} splits={splits} causal={causal} meta={meta} page={page} "
          f"axes={kaxis}/{vaxis}", flush=True)
    kc, vc = _caches(w, data, meta, page, kaxis=kaxis, vaxis=vaxis)
    out = _gpu.run_attention(w, data, kc, vc, corr=corr, path="short", splits=splits, causal=causal)
    ref = oracle_problem(orc, w, corr, data=data, causal=causal, meta=meta, kaxis=kaxis, vaxis=vaxis).attention()
    _gpu.check(_gpu.out_rows(out), ref)
    return out


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("corr", ["off", "taylor"])
def test_parity(orc, case, corr):
    _compare(orc, CASES[case], corr)


@pytest.mark.parametrize("kbits,vbits", [(2, 2), (2, 4), (4, 2), (4, 4)])
@pytest.mark.parametrize("group", [32, 64, 128])
def test_bits_and_groups(orc, kbits, vbits, group):
    w = GQA.scaled(B=2, Hq=8, Hkv=2, Nq=2, Ncur=3, Nc=600, group=group, kbits=kbits, vbits=vbits)
    _compare(orc, w, "taylor")


@pytest.mark.parametrize("splits", [1, 3, 7, 40])
def test_split_counts(orc, splits):
    _compare(orc, CASES["gqa_decode_g64"], "taylor", splits=splits)


@pytest.mark.parametrize("splits", [0, 5])
def test_causal(orc, splits):
    w = GQA.scaled(B=2, Hq=8, Hkv=2, Nq=4, Ncur=9, Nc=500, group=64)
    _compare(orc, w, "taylor", splits=splits, causal=True)


@pytest.mark.parametrize("meta", ["f16", "bf16"])
@pytest.mark.parametrize("case", ["gqa_chunk4_g32", "outliers_decode"])
def test_meta16(orc, meta, case):
    _compare(orc, CASES[case], "taylor", meta=meta)


@pytest.mark.parametrize("meta", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("page", [32, 128])
def test_paged_matches_contiguous(orc, meta, page):
    """Pages of 32 (one key block) and 128 tokens, shuffled: bit-identical to
    the contiguous cache, and within the bar of the oracle."""
    import _gpu
    w = GQA.scaled(B=3, Hq=8, Hkv=2, Nq=2, Ncur=2, Nc=700, group=32 if page == 32 else 64)
    data = W.generate(w)
    a = _compare(orc, w, "taylor", meta=meta, page=page)
    kc, vc = _caches(w, data, meta)
    b = _gpu.run_attention(w, data, kc, vc, corr="taylor", path="short")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_general_kernel_agrees(orc):
    """path = long sends the same call to the general kernel (its token-axis
    instances): both kernels meet the oracle's bar on the same inputs."""
    import _gpu
    w = H24.scaled(B=1, Hq=2, Hkv=2, Nq=16, Ncur=16, Nc=640, group=64)
    data = W.generate(w)
    kc, vc = _caches(w, data)
    ref = oracle_problem(orc, w, "taylor", data=data, kaxis="tokens", vaxis="dim").attention()
    for path in ("short", "long"):
        out = _gpu.run_attention(w, data, kc, vc, corr="taylor", path=path)
        _gpu.check(_gpu.out_rows(out), ref, f"{path}: ")


def test_offsets_far_from_zero(orc):
    """Keys with a shared per-channel offset of +-150 (logits in the hundreds): q.z is
    summed in fp32, so the offset costs no precision."""
    import _gpu
    w = GQA.scaled(B=1, Hq=8, Hkv=2, Nq=2, Ncur=2, Nc=800, group=64)
    data = W.generate(w)
    rng = np.random.default_rng(11)
    off = rng.choice([-150.0, 150.0], size=(1, w.Hkv, 1, w.d)).astype(np.float32)
    data["kc"] = (data["kc"] + off).astype(np.float32)
    data["k"] = W.bf16_bits(W.bf16_to_f32(data["k"]) + off)
    print(f"[tokens short] offsets +-150: Nc={w.Nc}", flush=True)
    kc, vc = _caches(w, data)
    out = _gpu.run_attention(w, data, kc, vc, corr="taylor", path="short")
    ref = oracle_problem(orc, w, "taylor", data=data, kaxis="tokens", vaxis="dim").attention()
    _gpu.check(_gpu.out_rows(out), ref)


VAXES = [("tokens", "tokens"), ("dim", "tokens")]


@pytest.mark.parametrize("axes", VAXES)
@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("corr", ["off", "taylor"])
def test_values_along_tokens(orc, axes, case, corr):
    _compare(orc, CASES[case], corr, kaxis=axes[0], vaxis=axes[1])


@pytest.mark.parametrize("axes", VAXES)
@pytest.mark.parametrize("kbits,vbits", [(2, 2), (2, 4), (4, 2), (4, 4)])
@pytest.mark.parametrize("group", [32, 64, 128])
def test_values_along_tokens_bits_and_groups(orc, axes, kbits, vbits, group):
    w = GQA.scaled(B=2, Hq=8, Hkv=2, Nq=2, Ncur=3, Nc=600, group=group, kbits=kbits, vbits=vbits)
    _compare(orc, w, "taylor", kaxis=axes[0], vaxis=axes[1])


@pytest.mark.parametrize("axes", VAXES)
@pytest.mark.parametrize("splits,causal", [(3, False), (40, False), (0, True), (5, True)])
def test_values_along_tokens_splits_causal(orc, axes, splits, causal):
    w = GQA.scaled(B=2, Hq=8, Hkv=2, Nq=4, Ncur=9, Nc=500, group=64)
    _compare(orc, w, "taylor", splits=splits, causal=causal, kaxis=axes[0], vaxis=axes[1])


@pytest.mark.parametrize("axes", VAXES)
@pytest.mark.parametrize("page", [32, 128])
def test_values_along_tokens_paged(orc, axes, page):
    import _gpu
    w = GQA.scaled(B=3, Hq=8, Hkv=2, Nq=2, Ncur=2, Nc=700, group=32 if page == 32 else 64)
    data = W.generate(w)
    a = _compare(orc, w, "taylor", page=page, kaxis=axes[0], vaxis=axes[1])
    kc, vc = _caches(w, data, kaxis=axes[0], vaxis=axes[1])
    b = _gpu.run_attention(w, data, kc, vc, corr="taylor", path="short")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("meta", ["f16", "bf16"])
def test_values_along_tokens_meta16_general(orc, meta):
    """16-bit metadata with values along the tokens stays on the general kernel."""
    _compare(orc, CASES["gqa_chunk4_g32"], "taylor", meta=meta, kaxis="tokens", vaxis="tokens")


# More than 16 query rows per KV head: the 32-row tiles (row groups of 32).
ROWS32 = {
    "gqa_rows20_g64": GQA.scaled(B=2, Hq=8, Hkv=2, Nq=5, Ncur=5, Nc=900, group=64),
    "gqa_rows32_g32": GQA.scaled(B=2, Hq=8, Hkv=2, Nq=8, Ncur=8, Nc=700, group=32),
    "gqa_rows64_g128": GQA.scaled(B=1, Hq=8, Hkv=2, Nq=16, Ncur=16, Nc=1100, group=128),
    "int4_rows40_ragged": H24.scaled(B=1, Hq=2, Hkv=2, Nq=40, Ncur=23, Nc=513, group=64),
    "outliers_rows24": OUT.scaled(Hq=4, Hkv=2, Nq=12, Ncur=12, Nc=800, group=64),
    "longvideo_rows17": LV.scaled(Hq=1, Hkv=1, Nq=17, Ncur=17, Nc=1000, group=64),
    "small_cache_rows24": GQA.scaled(B=2, Hq=8, Hkv=2, Nq=6, Ncur=6, Nc=20, group=32),
}
AXES3 = [("tokens", "dim"), ("tokens", "tokens"), ("dim", "tokens")]


@pytest.mark.parametrize("axes", AXES3)
@pytest.mark.parametrize("case", sorted(ROWS32))
@pytest.mark.parametrize("corr", ["off", "taylor"])
def test_rows32(orc, axes, case, corr):
    _compare(orc, ROWS32[case], corr, kaxis=axes[0], vaxis=axes[1])


@pytest.mark.parametrize("axes", AXES3)
@pytest.mark.parametrize("kbits,vbits", [(2, 4), (4, 2)])
def test_rows32_bits_splits_causal(orc, axes, kbits, vbits):
    w = GQA.scaled(B=2, Hq=8, Hkv=2, Nq=8, Ncur=11, Nc=600, group=64, kbits=kbits, vbits=vbits)
    _compare(orc, w, "taylor", splits=3, kaxis=axes[0], vaxis=axes[1])
    _compare(orc, w, "taylor", splits=0, causal=True, kaxis=axes[0], vaxis=axes[1])


@pytest.mark.parametrize("axes", AXES3)
def test_rows32_paged_matches_contiguous(orc, axes):
    import _gpu
    w = GQA.scaled(B=3, Hq=8, Hkv=2, Nq=6, Ncur=6, Nc=700, group=64)
    data = W.generate(w)
    a = _compare(orc, w, "taylor", page=128, kaxis=axes[0], vaxis=axes[1])
    kc, vc = _caches(w, data, kaxis=axes[0], vaxis=axes[1])
    b = _gpu.run_attention(w, data, kc, vc, corr="taylor", path="short")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_rows_above_64_forced_short(orc):
    """A forced short path at 100 rows per KV head: four row groups."""
    w = H24.scaled(B=1, Hq=2, Hkv=2, Nq=100, Ncur=100, Nc=400, group=64)
    _compare(orc, w, "taylor", kaxis="tokens", vaxis="tokens")


@pytest.mark.parametrize("meta", ["f16", "bf16"])
def test_rows32_meta16_general(orc, meta):
    """16-bit metadata above 16 rows stays on the general kernel."""
    _compare(orc, ROWS32["gqa_rows20_g64"], "taylor", meta=meta, kaxis="tokens", vaxis="dim")


@pytest.mark.parametrize("axes", AXES3)
def test_prefill_auto_path(orc, axes):
    """300 rows per KV head with the path left to the library: caches grouped
    along the tokens run on the short-query tiles (ten row groups), not on
    the general kernel."""
    import _gpu
    w = H24.scaled(B=1, Hq=2, Hkv=2, Nq=300, Ncur=300, Nc=700, group=64)
    data = W.generate(w)
    print(f"[tokens prefill] axes={axes} Nq={w.Nq} Nc={w.Nc}", flush=True)
    kc, vc = _caches(w, data, kaxis=axes[0], vaxis=axes[1])
    out = _gpu.run_attention(w, data, kc, vc, corr="taylor", path="auto")
    ref = oracle_problem(orc, w, "taylor", data=data, kaxis=axes[0], vaxis=axes[1]).attention()
    _gpu.check(_gpu.out_rows(out), ref)
