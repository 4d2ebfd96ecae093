"""kv_attention_corrected_static (no allocation, a static scratch array in the
library) against kv_attention_corrected on the same inputs, through the C
ABI: two calls in a row, the second with a smaller input, on each kernel
path.  Where both entry points take the same plan the outputs are
bit-identical; where the static one lowers the split count to fit its
array, the outputs are held to the parity bar against each other and
against the oracle on sampled rows."""
import ctypes as C

import numpy as np
import pytest
import torch

from bit_kv_cache_03_amd import kvq
from bit_kv_cache_03_amd import workloads as W
from _problems import oracle_problem

pytestmark = pytest.mark.gpu


def _inputs(w):
    import _gpu
    data = W.generate(w)
    kc = _gpu.build_cache(w, data["kc"], w.kbits)
    vc = _gpu.build_cache(w, data["vc"], w.vbits)
    q = _gpu.as_bf16_dev(data["q"])
    k = _gpu.as_bf16_dev(data["k"]) if w.Ncur > 0 else None
    v = _gpu.as_bf16_dev(data["v"]) if w.Ncur > 0 else None
    return data, q, k, v, kc, vc


def _both(w, corr, path):
    """Outputs of the workspace entry point and of the static one."""
    data, q, k, v, kc, vc = _inputs(w)
    ref = kvq.attention(q, k, v, kc, vc, w.Nc, corr=corr, path=path)
    out = torch.full_like(q, float("nan"))
    a = kvq.make_args(q, k, v, kc, vc, w.Nc, out, corr=corr, path=path)
    print(f"[static] B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} Nq={w.Nq} Ncur={w.Ncur} Nc={w.Nc} corr={corr} "
          f"path={path} workspace of the other entry point={kvq.workspace_size(a)}", flush=True)
    st = kvq.lib.kv_attention_corrected_static(C.byref(a), torch.cuda.current_stream().cuda_stream)
    assert st == kvq.KV_OK, kvq.lib.kv_status_string(st)
    torch.cuda.synchronize()
    return data, ref, out


PAIRS = {
    # (first call, second smaller call, correction, path)
    "throughput": (W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=2, Hq=8, Hkv=2, Nq=100, Ncur=100, Nc=700),
                   W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=1, Hq=8, Hkv=2, Nq=40, Ncur=40, Nc=300),
                   "taylor", "long"),
    "short": (W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=2, Hq=8, Hkv=2, Nq=4, Ncur=20, Nc=900),
              W.WORKLOADS["gqa_prefill_b16_cache32k"].scaled(B=1, Hq=8, Hkv=2, Nq=2, Ncur=7, Nc=400),
              "taylor", "short"),
    "general": (W.WORKLOADS["tiny_d64_int2"].scaled(Hq=4, Hkv=2, Nq=90, Ncur=90, Nc=520),
                W.WORKLOADS["tiny_d64_int2"].scaled(Hq=2, Hkv=1, Nq=30, Ncur=10, Nc=200),
                "exact", "auto"),
}


@pytest.mark.parametrize("kernel", sorted(PAIRS))
def test_static_matches_workspace_entry(kernel):
    big, small, corr, path = PAIRS[kernel]
    for w in (big, small):
        _, ref, out = _both(w, corr, path)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_static_lowers_the_split_to_fit(orc):
    """300 KV heads of 100 rows: the workspace entry point splits the 44
    tail units 5 ways (79 MB of partials, more than the 64 MiB array); the
    static one runs them unsplit.  Then a smaller call reuses the array."""
    import _gpu
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the split plan under test assumes 256 CUs")
    w = W.WORKLOADS["h24_int4_cache16k"].scaled(Hq=300, Hkv=300, Nq=100, Ncur=100, Nc=500)
    data, ref, out = _both(w, "taylor", "auto")
    got, want = _gpu.out_rows(out), _gpu.out_rows(ref)
    _gpu.check(got, want, "static vs workspace entry: ")
    rows = np.array([h * w.Nq + j for h in (0, 255, 256, 299) for j in (0, 57, 99)], dtype=np.int64)
    _gpu.check(got[rows], oracle_problem(orc, w, "taylor", data=data).attention(rows=rows), "static vs oracle: ")
    small = w.scaled(Hq=20, Hkv=20, Nq=90, Ncur=90, Nc=300)
    _, ref, out = _both(small, "taylor", "auto")
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
