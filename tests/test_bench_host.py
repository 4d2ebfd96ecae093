"""Host-side arithmetic of bench.py: the algorithmic work counts behind the
roofline figures (no GPU)."""
import importlib.util
import os

import pytest
from torch.nn.attention.bias import causal_lower_right

from bit_kv_cache_03_amd import workloads as W

_spec = importlib.util.spec_from_file_location(
    "bench", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


@pytest.mark.parametrize("nq,ncur", [(1, 37), (5, 9), (6, 6), (7, 4), (300, 300), (4096, 4096)])
def test_visible_pairs_match_lower_right_mask(nq, ncur):
    w = W.WORKLOADS["h24_int4_cache16k"].scaled(Nq=nq, Ncur=ncur)
    assert bench.visible_current_pairs(w, False) == nq * ncur
    assert bench.visible_current_pairs(w, True) == int(causal_lower_right(nq, ncur)._materialize().sum())


def test_flops_and_bytes_of_the_default_workload():
    w = W.WORKLOADS["h24_int4_cache16k"]
    # 4 d flops per (query, key) pair over the cache and the chunk
    assert bench.attention_flops(w) == 4.0 * 128 * 24 * 4096 * (16384 + 4096)
    # square chunk under the mask: Nq (Nq + 1) / 2 current pairs per head
    assert bench.attention_flops(w, causal=True) == 4.0 * 128 * 24 * (4096 * 16384 + 4096 * 4097 // 2)
    # INT4 K and V codes (64 + 64 bytes) plus fp32 step and zero of 2 groups for K and V (32 bytes)
    assert bench.packed_bytes(w) == 24 * 16384 * 160
    # binary16 step and zero: 16 bytes of metadata per token instead of 32
    assert bench.packed_bytes(w, 2) == 24 * 16384 * 144
    # K grouped along the tokens (group 64): 2 x 128 fp32 values per 64 tokens (16 bytes per token)
    assert bench.packed_bytes(w, 4, "tokens", "dim") == 24 * 16384 * 128 + 24 * 256 * 2 * 128 * 4 + 24 * 16384 * 16


def test_default_workload_is_the_largest_single_gpu_one():
    """The timed default is the workload with the most algorithmic flops."""
    flops = {n: bench.attention_flops(w) for n, w in W.WORKLOADS.items()}
    assert bench.DEFAULT_WORKLOAD == max(flops, key=flops.get) == "gqa_prefill_b16_cache32k"
    assert bench.MALL_EVICT_BYTES >= 512 << 20


def test_dtype_names_the_arithmetic_of_the_kernel():
    w = W.WORKLOADS["gqa_prefill_b16_cache32k"]
    assert bench.arithmetic(w, "taylor", 0, "dim", "dim")["dtype"] == "fp16"
    assert bench.arithmetic(w, "exact", 0, "dim", "dim")["dtype"] == "bf16"
    assert bench.arithmetic(W.WORKLOADS["tiny_d64_int2"], "off", 0, "dim", "dim")["dtype"] == "bf16"
    # caches grouped along the tokens: the short-query kernels (fp16) where they serve the call
    assert bench.arithmetic(w, "taylor", 0, "tokens", "dim")["dtype"] == "fp16"
    assert bench.arithmetic(w, "taylor", 0, "tokens", "tokens", "f32")["dtype"] == "fp16"
    assert bench.arithmetic(w, "taylor", 0, "tokens", "dim", "f32", "long")["dtype"] == "bf16"
    assert bench.arithmetic(w, "taylor", 0, "tokens", "dim", "f16")["dtype"] == "bf16"  # 2048 rows per KV head
    assert bench.arithmetic(w.scaled(Nq=4, Ncur=4), "taylor", 0, "tokens", "dim", "f16")["dtype"] == "fp16"
    assert bench.arithmetic(w.scaled(Nq=4, Ncur=4), "taylor", 0, "tokens", "tokens", "bf16")["dtype"] == "bf16"
    assert "subnormals" in bench.arithmetic(w, "taylor", 0, "tokens", "dim")["dtype_detail"]
