"""Benchmark of the corrected INT2/INT4 KV-cache attention hot path on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--corr taylor]

One step = the whole hot path over one chunk of synthetic input, inputs
already resident in HBM:
  - kv_attention_corrected: the current chunk's queries against the Nc
    cached (INT2/INT4, dequantised in-kernel) tokens and the bf16 current
    chunk, Jensen-bias correction on cached scores, one online softmax;
  - the finished chunk's K and V quantised and appended to the cache at
    rows [Nc, Nc + Ncur) (rows the attention of this step does not read,
    so every step does identical work): by default inside the same call
    (append = 1), with --append separate by two kv_quantize calls.
Prints ONE JSON line.  `value` is cached-key tokens x queries per second of
whole steps; the attention kernel's own duration (HIP events on the stream
it runs on) gives the roofline figure.  The CPU oracle, timed on a bounded
sample of the same workload on this host's cores, is the `cpu_baseline`.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from bit_kv_cache_03_amd import workloads as W  # noqa: E402

# the largest workload that fits one GPU (4.47e12 flop, a 537 MB packed cache)
DEFAULT_WORKLOAD = "gqa_prefill_b16_cache32k"
MALL_EVICT_BYTES = 512 << 20  # > the 256 MB MALL: written between HBM-graded launches
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "cached-key tokens\u00b7queries/s (TFLOP/s eff.) and packed-KV HBM GB/s vs roofline"
# every source the library is built from (the hash names the kernels a
# stored counter run measured)
KERNEL_SOURCES = sorted(glob.glob(os.path.join(ROOT, "bit_kv_cache_03_amd", "csrc", "*.hip")) +
                        glob.glob(os.path.join(ROOT, "bit_kv_cache_03_amd", "csrc", "*.h")) +
                        glob.glob(os.path.join(ROOT, "bit_kv_cache_03_amd", "csrc", "*.cpp")))


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def packed_bytes(w, meta_bytes: int = 4, kaxis: str = "dim", vaxis: str = "dim") -> int:
    """Algorithmic bytes of the packed cache read by one attention call:
    codes of K and V plus step and zero of both (fp32: 4 bytes each,
    binary16: 2), over Nc tokens; a tensor grouped along the tokens holds
    d steps and zero points per ceil(Nc / group) tokens instead of d / group
    per token."""
    codes = w.B * w.Hkv * w.Nc * (w.d * (w.kbits + w.vbits) // 8)
    meta = 0
    for axis in (kaxis, vaxis):
        groups = -(-w.Nc // w.group) if axis == "tokens" else w.Nc * (w.d // w.group) // w.d
        meta += w.B * w.Hkv * 2 * groups * w.d * meta_bytes
    return codes + meta


def visible_current_pairs(w, causal: bool) -> int:
    """(query row, current key) pairs per head: all of them, or under the
    end-aligned causal mask those with key i <= j + Ncur - Nq."""
    if not causal:
        return w.Nq * w.Ncur
    j = np.arange(w.Nq)
    return int(np.clip(j + w.Ncur - w.Nq + 1, 0, w.Ncur).sum())


def attention_flops(w, causal: bool = False) -> float:
    """Algorithmic flops: Q K^T and P V over the visible (query, key) pairs
    of both segments (4 d per pair)."""
    return 4.0 * w.d * w.B * w.Hq * (w.Nq * w.Nc + visible_current_pairs(w, causal))


def call_options(args) -> dict:
    """The options of the timed attention call besides the workload."""
    return {"nq": args.nq, "corr": args.corr, "path": args.path, "causal": args.causal,
            "page_size": args.page_size, "meta": args.meta, "kaxis": args.kaxis, "vaxis": args.vaxis,
            "append": args.append}


def traffic_from_profiles(w, sha: str, options: dict):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    runs, if they were taken on the current kernel source with the same call
    options."""
    path = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sha") != sha or t.get("options") != options:
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, data, corr: str, target_s: float = 12.0, causal: bool = False, meta: str = "f32",
                 kaxis: str = "dim", vaxis: str = "dim"):
    """The oracle as it stands, on a bounded sample of query rows (all heads,
    rows spread over the chunk), with the quantize of the chunk prorated."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    kc = oracle.quantize(data["kc"], w.kbits, w.group, meta=meta, axis=kaxis)
    vc = oracle.quantize(data["vc"], w.vbits, w.group, meta=meta, axis=vaxis)
    qb = lambda x: x if x.dtype == np.uint16 else W.bf16_bits(x)
    prob = oracle.Problem(qb(data["q"]), qb(data["k"]), qb(data["v"]), kc, vc, w.Nc, w.kbits, w.vbits,
                          w.group, corr=corr, causal=causal, kaxis=kaxis, vaxis=vaxis)
    total = prob.rows_total()
    t0 = time.perf_counter()
    oracle.quantize(data["k"], w.kbits, w.group, meta=meta, axis=kaxis)
    oracle.quantize(data["v"], w.vbits, w.group, meta=meta, axis=vaxis)
    t_quant = time.perf_counter() - t0
    # grow a calibration sample until it runs for a second, then size the
    # timed sample for about target_s seconds
    n_cal = max(4 * threads, 16)
    while True:
        cal = np.linspace(0, total - 1, num=min(n_cal, total)).astype(np.int64)
        t0 = time.perf_counter()
        prob.attention(rows=cal, threads=threads)
        t_cal = time.perf_counter() - t0
        if t_cal >= 1.0 or cal.size >= total:
            break
        n_cal = int(n_cal * min(8.0, max(2.0, 1.2 / max(t_cal, 1e-3))))
    per_row = t_cal / cal.size
    n = int(min(total, max(cal.size, target_s / per_row)))
    rows = np.linspace(0, total - 1, num=n).astype(np.int64)
    t0 = time.perf_counter()
    prob.attention(rows=rows, threads=threads)
    t_rows = time.perf_counter() - t0
    t = t_rows + t_quant * n / total
    return {"value": n * w.Nc / t, "unit": "cached-key tokens·queries/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} of {total} query rows (every {total / n:.1f}th, all heads) of {w.name}, "
                      f"fp64 oracle attention with {corr} correction over all {w.Nc}+{w.Ncur} keys"
                      f"{' (causal mask on the current chunk)' if causal else ''}, "
                      f"plus the chunk's quantize prorated; {t:.1f} s wall on {threads} threads"}


def arithmetic(w, corr: str, page_size: int, kaxis: str, vaxis: str, meta: str = "f32", path: str = "auto") -> dict:
    """The arithmetic the attention call computes in, by the kernel that
    serves it: head dim 128 with correction off or Taylor and pages of at
    least one 32/64-key tile run the fp16 kernels (caches grouped along the
    tokens on the short-query path: any metadata with keys alone along the
    tokens at up to 16 rows per KV head, fp32 metadata otherwise); the rest
    runs the general kernel (bf16 hi + lo keys)."""
    tok = "tokens" in (kaxis, vaxis)
    rows = w.Nq * (w.Hq // w.Hkv)
    fp16 = w.d == 128 and corr != "exact" and (page_size == 0 or page_size >= 32)
    if tok:
        fp16 = fp16 and path != "long" and (meta == "f32" or (rows <= 16 and vaxis == "dim"))
    if fp16:
        keys = ("keys grouped along the tokens enter as their codes (exact fp16 subnormals c 2^-24) against queries "
                "scaled per channel by the token group's steps, with q.z and the per-channel Taylor bias in fp32; "
                if kaxis == "tokens" else
                "keys and values scaled by powers of two into the fp16 range; the correction and running-max step "
                "on bf16 MFMA (hi + lo splits); ")
        return {"dtype": "fp16",
                "dtype_detail": "Q K^T and P V on fp16 MFMA with fp32 accumulation, " + keys +
                                "softmax in fp32; bf16 inputs and outputs; INT%d keys / INT%d values dequantised "
                                "in-kernel" % (w.kbits, w.vbits)}
    return {"dtype": "bf16",
            "dtype_detail": "Q K^T on bf16 MFMA with keys split into bf16 hi + lo parts, P V on fp16 MFMA, fp32 "
                            "accumulation and softmax; bf16 inputs and outputs"}


class ClockProbe:
    """Shader (sclk) and memory (mclk) clocks of the GPU this process uses
    (amdsmi, matched by PCI address).  Opened before the timed steps, so that
    sample() costs little and lands while the enqueued steps still run; the
    record is informative only (None fields where amdsmi is unavailable)."""

    def __init__(self):
        self.h, self.err = None, None
        try:
            import amdsmi
            import torch
            pr = torch.cuda.get_device_properties(torch.cuda.current_device())
            self.bdf = "%04x:%02x:%02x.0" % (pr.pci_domain_id, pr.pci_bus_id, pr.pci_device_id)
            amdsmi.amdsmi_init()
            self.amdsmi = amdsmi
            self.h = amdsmi.amdsmi_get_processor_handle_from_bdf(self.bdf)
        except Exception as e:
            self.err = f"{type(e).__name__}: {e}"

    def sample(self, done):
        """Poll the clocks every ~2 ms until done() (the timed steps have
        finished); the median and the largest reading of each."""
        if self.h is None:
            return {"error": self.err}
        try:
            a = self.amdsmi
            gs, ms = [], []
            while True:
                finished = done()
                gs.append(a.amdsmi_get_clock_info(self.h, a.AmdSmiClkType.SYS))
                ms.append(a.amdsmi_get_clock_info(self.h, a.AmdSmiClkType.MEM))
                if finished or len(gs) >= 2000:
                    break
                time.sleep(0.002)
            g = [x.get("clk") for x in gs if isinstance(x.get("clk"), (int, float))]
            m = [x.get("clk") for x in ms if isinstance(x.get("clk"), (int, float))]
            return {"sclk_mhz_median": float(np.median(g)) if g else None, "sclk_mhz_max": max(g) if g else None,
                    "sclk_max_mhz": gs[0].get("max_clk"), "mclk_mhz_median": float(np.median(m)) if m else None,
                    "mclk_max_mhz": ms[0].get("max_clk"), "samples": len(gs), "bdf": self.bdf,
                    "source": "amdsmi, polled every ~2 ms from the enqueue of the timed steps to their end",
                    "note": "as amdsmi reports them: on the MI355X systems measured here the readings stay near "
                            "the idle level under load (a bf16 GEMM read 224 MHz on every XCD), so they are a "
                            "record, not the clock the kernels ran at"}
        except Exception as e:
            return {"error": f"{type(e).__name__}: {e}"}

    def close(self):
        if self.h is not None:
            try:
                self.amdsmi.amdsmi_shut_down()
            except Exception:
                pass


def copy_probe(nbytes: int, reps: int = 3):
    """A plain streaming kernel of known traffic (reads nbytes, writes
    nbytes: an elementwise negation), profiled beside the attention to scale
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def _counter_means(csv_path: str, counter: str, kernel_substrs) -> dict:
    """Mean per dispatch of one counter for each kernel whose name holds one
    of kernel_substrs (keyed by that substring)."""
    import csv
    vals = {}
    for r in csv.DictReader(open(csv_path)):
        hit = [k for k in kernel_substrs if k in r["Kernel_Name"]]
        if r["Counter_Name"] == counter and hit:
            vals.setdefault(hit[0], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel_substrs!r} in {csv_path}")
    return {k: float(np.mean(v)) for k, v in vals.items()}


# kernels one kv_attention_corrected call launches (pre-pass, attention, combine)
ATTENTION_CALL_KERNELS = ("key_scale_kernel", "attn_fast_kernel", "attn_short_kernel", "attn_tile_kernel",
                          "attn_combine_kernel", "tail_combine_kernel")


def write_traffic(w, pmc_dir: str, copy_bytes: int, options: dict):
    """HBM bytes per attention call from four rocprofv3 --pmc runs under
    pmc_dir (fetch/, write/: the bench; copy_fetch/, copy_write/: the copy
    probe): each kernel's mean counter per dispatch, scaled by bytes per
    KiB-reading of the plain copy, summed over the kernels of one call (the
    span bench times)."""
    f = lambda sub: os.path.join(pmc_dir, sub, "run_counter_collection.csv")
    fetch = _counter_means(f("fetch"), "FETCH_SIZE", ATTENTION_CALL_KERNELS)
    write = _counter_means(f("write"), "WRITE_SIZE", ATTENTION_CALL_KERNELS)
    cf = copy_bytes / (1024.0 * sum(_counter_means(f("copy_fetch"), "FETCH_SIZE", ("neg",)).values()))
    cw = copy_bytes / (1024.0 * sum(_counter_means(f("copy_write"), "WRITE_SIZE", ("neg",)).values()))
    per_kernel = {k: {"fetch_bytes": 1024.0 * fetch.get(k, 0.0) * cf, "write_bytes": 1024.0 * write.get(k, 0.0) * cw}
                  for k in sorted(set(fetch) | set(write))}
    t = {"workload": w.name, "options": options, "kernel_sha": kernel_sha(), "copy_bytes": copy_bytes,
         "fetch_factor": cf,
         "write_factor": cw, "per_kernel": per_kernel,
         "bytes_per_launch": sum(v["fetch_bytes"] + v["write_bytes"] for v in per_kernel.values()),
         "algorithmic_packed_bytes": packed_bytes(w, 4 if options["meta"] == "f32" else 2, options["kaxis"],
                                                  options["vaxis"])}
    out = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    with open(out, "w") as fh:
        json.dump(t, fh, indent=1)
    print(json.dumps(t))


def diag_bench(args, w, corr, data, dev, q, k, kc):
    """Time kv_attention_diagnostics (correction off and the workload's mode)
    on the full workload and summarise the statistics over all rows."""
    import ctypes as C
    import torch
    from bit_kv_cache_03_amd import kvq
    kref = dev(data["kc"])
    stream = torch.cuda.current_stream()
    rows = w.B * w.Hq * w.Nq
    res = {}
    for mode in dict.fromkeys(("off", corr)):
        rec = torch.empty((rows, kvq.DIAG_ROW_WORDS), dtype=torch.int32, device="cuda")
        a = kvq.make_diag_args(q, k, kref, kc, w.Nc, rec, corr=mode, causal=args.causal)
        call = lambda: kvq._check(kvq.lib.kv_attention_diagnostics(C.byref(a), stream.cuda_stream),
                                  "kv_attention_diagnostics")
        for _ in range(args.warmup):
            call()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for e0, e1 in evs:
            e0.record(stream)
            call()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
        r = rec.cpu().numpy()
        st = r[:, :5].view(np.float32).astype(np.float64)
        top = r[:, 5:15].reshape(-1, 2, 5)
        recall = np.mean([len(set(a[a >= 0]) & set(b[b >= 0])) / max(1, int((a >= 0).sum())) for a, b in top])
        res[mode] = {"ms": ms, "mass_q": float(st[:, 3].mean()), "kl": float(st[:, 4].mean()),
                     "top1_drift": float((top[:, 0, 0] != top[:, 1, 0]).mean()), "top5_recall": float(recall),
                     "mass_ref": float(st[:, 2].mean())}
    # algorithmic work: 2d flops per visible (row, key) pair for each score
    # set; the current chunk's scores are shared by both sets
    pairs_c = w.B * w.Hq * w.Nq * w.Nc
    pairs_u = w.B * w.Hq * visible_current_pairs(w, args.causal)
    flops = 2.0 * w.d * (2 * pairs_c + pairs_u)
    ms = res[corr]["ms"]
    line = {
        "metric": "attention-balance diagnostics (kv_attention_diagnostics)",
        "workload": w.name, "corr": corr, "causal": args.causal, "rows": rows, "steps": args.steps,
        "ms": ms, "roofline": {"bound": "mfma", "achieved": flops / (ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                               "unit": "TFLOP/s", "frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "mass_ref": res[corr]["mass_ref"],
        "modes": {m: {k: v for k, v in d.items() if k != "mass_ref"} for m, d in res.items()},
        "data": "synthetic: seeded, the workload's key structure; reference = the cached keys before quantisation",
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(W.WORKLOADS))
    ap.add_argument("--corr", default=None, choices=["off", "taylor", "exact"])
    ap.add_argument("--path", default="auto", choices=["auto", "long", "short"])
    ap.add_argument("--nq", type=int, default=0, help="override query rows (and current chunk) per head")
    ap.add_argument("--causal", action="store_true", help="end-aligned causal mask within the current chunk")
    ap.add_argument("--page-size", type=int, default=0,
                    help="paged cache layout with pages of this many tokens (shuffled page table)")
    ap.add_argument("--meta", default="f32", choices=["f32", "f16", "bf16"],
                    help="storage type of the caches' step and zero point")
    ap.add_argument("--kaxis", default="dim", choices=["dim", "tokens"],
                    help="K cache groups along the head dimension or along the tokens (per channel)")
    ap.add_argument("--vaxis", default="dim", choices=["dim", "tokens"], help="the same for V")
    ap.add_argument("--diag", action="store_true",
                    help="time kv_attention_diagnostics and report the attention-balance statistics instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-overhead", action="store_true", help="skip the correction-off timing")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    ap.add_argument("--traffic", default=None, metavar="PMC_DIR",
                    help="only turn rocprofv3 FETCH_SIZE/WRITE_SIZE runs into profiles/traffic_<workload>.json")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--append", default="fused", choices=["fused", "separate"],
                    help="append the chunk to the cache inside the attention call, or by kv_quantize after it")
    ap.add_argument("--evict", default="auto", choices=["auto", "on", "off"],
                    help="pass over a 512 MiB buffer between timed steps so that no launch finds the cache in the "
                         "MALL (auto: on for HBM-graded runs, i.e. at most 64 query rows per KV head)")
    ap.add_argument("--evict-by", default="read", choices=["read", "write"],
                    help="how the eviction passes over the 512 MiB buffer: a read (leaves clean lines) or a write "
                         "(leaves dirty lines whose write-back falls inside the next timed step)")
    args = ap.parse_args()
    if "tokens" in (args.kaxis, args.vaxis):
        args.append = "separate"  # the fused append takes caches grouped along the head dimension
    if args.traffic:
        write_traffic(W.WORKLOADS[args.workload], args.traffic, args.copy_bytes, call_options(args))
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import torch
    from bit_kv_cache_03_amd import kvq

    w = W.WORKLOADS[args.workload]
    if args.nq:
        w = w.scaled(Nq=args.nq, Ncur=args.nq)
    corr = args.corr or w.corr
    data = W.generate(w)
    dev = lambda x: (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if x.dtype == np.uint16
                     else torch.from_numpy(W.bf16_bits(x).view(np.int16)).view(torch.bfloat16)).cuda()
    q, k, v = dev(data["q"]), dev(data["k"]), dev(data["v"])
    cap = w.Nc + w.Ncur
    if "tokens" in (args.kaxis, args.vaxis):
        cap = -(-cap // w.group) * w.group  # whole token groups
    if args.page_size:
        # pages of a shuffled pool: every (sequence, block) on a page drawn at random
        ps = args.page_size
        cap = (cap + ps - 1) // ps * ps
        npages = w.B * (cap // ps)
        perm = np.random.default_rng(11).permutation(npages).astype(np.int32).reshape(w.B, cap // ps)
        table = torch.from_numpy(perm).cuda()
        paged = dict(page_table=table, page_size=ps, num_pages=npages)
    else:
        paged = {}
    kc = kvq.QCache(w.B, w.Hkv, cap, w.d, w.kbits, w.group, meta=args.meta, axis=args.kaxis, **paged)
    vc = kvq.QCache(w.B, w.Hkv, cap, w.d, w.vbits, w.group, meta=args.meta, axis=args.vaxis, **paged)
    # the cache content does not depend on how it is appended (quantisation
    # is per token), so short chunks are appended in >= 4096-token calls
    chunk = max(w.Ncur, 4096)
    for off in range(0, w.Nc, chunk):
        n = min(chunk, w.Nc - off)
        kvq.quantize(dev(np.ascontiguousarray(data["kc"][:, :, off:off + n])), kc, off)
        kvq.quantize(dev(np.ascontiguousarray(data["vc"][:, :, off:off + n])), vc, off)
    if args.diag:
        diag_bench(args, w, corr, data, dev, q, k, kc)
        return
    out = torch.empty_like(q)
    # one workspace for the timed mode and the correction-off comparison
    # (which may take another kernel: the exact form runs on the general one)
    ws_bytes = max(kvq.workspace_size(kvq.make_args(q, k, v, kc, vc, w.Nc, out, corr=c, path=args.path,
                                                    causal=args.causal)) for c in (corr, "off"))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    fused = args.append == "fused"
    args_c = kvq.make_args(q, k, v, kc, vc, w.Nc, out, corr=corr, path=args.path, workspace=ws,
                           causal=args.causal, append=fused)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    import ctypes as C

    def attention(a):
        st = kvq.lib.kv_attention_corrected(C.byref(a), sp)
        if st != 0:
            raise kvq.KvqError(st, "kv_attention_corrected")

    def step(a, ev=None):
        if ev is not None:
            ev[0].record(stream)
        attention(a)
        if ev is not None:
            ev[1].record(stream)
        if not fused:
            kvq.quantize(k, kc, w.Nc, stream)
            kvq.quantize(v, vc, w.Nc, stream)

    # few query rows per KV head: the packed cache read bounds the kernel
    hbm_bound = w.rows_per_kvhead <= 64
    evict = args.evict == "on" or (args.evict == "auto" and hbm_bound)
    scratch = torch.empty(MALL_EVICT_BYTES // 4, dtype=torch.float32, device="cuda") if evict else None
    if scratch is not None:
        scratch.zero_()

    def evict_pass(buf, i):
        if args.evict_by == "read":
            buf.amax()
        else:
            buf.fill_(float(i))
    for _ in range(args.warmup):
        step(args_c)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    s_end = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    probe = ClockProbe()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        if scratch is not None:
            evict_pass(scratch, i)  # evicts the cache's lines from the MALL; outside the step's events
        step(args_c, evs[i])
        s_end[i].record(stream)
    t_end.record(stream)
    clocks = probe.sample(t_end.query)  # the steps above are still running: launches are asynchronous
    torch.cuda.synchronize()
    probe.close()
    wall = time.perf_counter() - wall0
    if scratch is None:
        ms_step = t_start.elapsed_time(t_end) / args.steps
    else:  # steps timed one by one, the eviction writes between them excluded
        ms_step = float(np.mean([a.elapsed_time(e) for (a, _), e in zip(evs, s_end)]))
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    quant_ms = ms_step - attn_ms
    del scratch

    overhead = append_overhead = None
    if not args.no_overhead:
        # interleaved so that drift hits all equally: the timed call, the
        # same with the correction off, and (fused) the same without append
        runs = {"on": args_c}
        if corr != "off":
            runs["off"] = kvq.make_args(q, k, v, kc, vc, w.Nc, out, corr="off", path=args.path, workspace=ws,
                                        causal=args.causal, append=fused)
        if fused:
            runs["plain"] = kvq.make_args(q, k, v, kc, vc, w.Nc, out, corr=corr, path=args.path, workspace=ws,
                                          causal=args.causal)
        for a in runs.values():
            for _ in range(args.warmup):
                attention(a)
        ev_runs = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(args.steps)] for n in runs}
        scratch = torch.empty(MALL_EVICT_BYTES // 4, dtype=torch.float32, device="cuda") if evict else None
        for i in range(args.steps):
            for n, a in runs.items():
                if scratch is not None:
                    evict_pass(scratch, i)
                ev_runs[n][i][0].record(stream); attention(a); ev_runs[n][i][1].record(stream)
        del scratch
        torch.cuda.synchronize()
        t = {n: float(np.median([a.elapsed_time(b) for a, b in e])) for n, e in ev_runs.items()}
        if "off" in t:
            overhead = t["on"] / t["off"] - 1.0
        if "plain" in t:
            append_overhead = t["on"] / t["plain"] - 1.0

    flops = attention_flops(w, args.causal)
    ckq = w.B * w.Hq * w.Nq * w.Nc
    achieved = flops / (attn_ms * 1e-3) / 1e12
    pbytes = packed_bytes(w, 4 if args.meta == "f32" else 2, args.kaxis, args.vaxis)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": pbytes / (attn_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    sha = kernel_sha()
    traffic = traffic_from_profiles(w, sha, call_options(args))
    line = {
        "metric": METRIC,
        "value": ckq / (ms_step * 1e-3),
        "unit": "cached-key tokens·queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        **arithmetic(w, corr, args.page_size, args.kaxis, args.vaxis, args.meta, args.path),
        "data": "synthetic: seeded N(0,1) q/k/v with the workload's key structure, bf16; cache INT%d/INT%d group %d%s" % (
            w.kbits, w.vbits, w.group, ({"f16": ", binary16 step/zero", "bf16": ", bfloat16 step/zero"}.get(args.meta, "")) +
            (f", K/V groups along {args.kaxis}/{args.vaxis}" if "tokens" in (args.kaxis, args.vaxis) else "")),
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "Nq": w.Nq,
                   "Ncur": w.Ncur, "Nc": w.Nc, "kbits": w.kbits, "vbits": w.vbits, "group": w.group,
                   "corr": corr, "path": args.path, "causal": args.causal, "page_size": args.page_size,
                   "meta": args.meta, "kaxis": args.kaxis, "vaxis": args.vaxis},
        "attention_ms": attn_ms,
        "quantize_ms": quant_ms,
        "tflops_eff": achieved,
        "packed_kv_gbs": pbytes / (attn_ms * 1e-3) / 1e9,
        "correction_overhead": overhead,
        "append": args.append,
        "append_overhead": append_overhead,
        "wall_s": wall,
        "kernel_sha": sha,
        "mall_evict_between_steps": evict,
        "mall_evict_by": args.evict_by if evict else None,
        "clocks": clocks,
        "roofline": dict(roof, frac=roof["achieved"] / roof["peak"], traffic=traffic),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, data, corr, causal=args.causal, meta=args.meta, kaxis=args.kaxis,
                                            vaxis=args.vaxis)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
