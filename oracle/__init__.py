"""CPU oracle for Jensen-bias-corrected low-bit KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
never calls into it and shares no code with it; a product path that reached
this module would be a bug.

The arithmetic lives in ``kvq_oracle.c`` (plain C, fp32 bit-exact quantizer,
fp64 attention); this module only builds and marshals.  Every function cites
the passage it follows in the C source.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

CORR = {"off": 0, "taylor": 1, "exact": 2}
META = {"f32": 0, "f16": 1, "bf16": 2}  # storage of the step and zero point


GCC_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-Wall", "-Wextra"]


def compile_source(src: str, out: str) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load(path: str):
    """Load a built oracle library and declare its signatures."""
    L = C.CDLL(path)
    i64, i32, dbl, vp = C.c_int64, C.c_int32, C.c_double, C.c_void_p
    L.kvo_quantize_f32.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp]
    L.kvo_quantize_bf16.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp]
    L.kvo_quantize_f32_meta.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp]
    L.kvo_quantize_bf16_meta.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp]
    L.kvo_quantize_tokens_f32_meta.argtypes = [vp, i64, i64, i32, i32, i32, i32, vp, vp, vp]
    L.kvo_quantize_tokens_bf16_meta.argtypes = [vp, i64, i64, i32, i32, i32, i32, vp, vp, vp]
    L.kvo_round_fp16.argtypes = [C.c_float]
    L.kvo_round_fp16.restype = C.c_float
    L.kvo_round_bf16.argtypes = [C.c_float]
    L.kvo_round_bf16.restype = C.c_float
    L.kvo_unpack.argtypes = [vp, i64, i32, i32, vp]
    L.kvo_pack.argtypes = [vp, i64, i32, i32, vp]
    L.kvo_dequant.argtypes = [vp, vp, vp, i64, i32, i32, i32, vp]
    L.kvo_logsinhc.argtypes = [dbl]
    L.kvo_logsinhc.restype = dbl
    L.kvo_bias_taylor.argtypes = [vp, vp, i32, i32, dbl]
    L.kvo_bias_taylor.restype = dbl
    L.kvo_bias_exact.argtypes = [vp, vp, i32, i32, dbl]
    L.kvo_bias_exact.restype = dbl
    L.kvo_logits.argtypes = [vp, i64, vp]
    L.kvo_attention.argtypes = [vp, vp, i64, vp, i32]
    L.kvo_attention_online.argtypes = [vp, i64, i64, vp, i64, i32, vp]
    L.kvo_diagnostics.argtypes = [vp, vp, vp, i64, vp, vp, i32]
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = _load(_LIB_PATH)
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


# --------------------------------------------------------------------------
# quantizer
# --------------------------------------------------------------------------

def quantize(x: np.ndarray, bits: int, group: int, meta: str = "f32", axis: str = "dim"):
    """Group-wise asymmetric quantization of the last axis of ``x``.

    ``x`` is float32 values, or uint16 bf16 bit patterns.  Returns
    ``(codes, step, zero)`` with codes packed LSB-first: shape
    ``x.shape[:-1] + (d*bits//8,)`` uint8, and step/zero of shape
    ``x.shape[:-1] + (d//group,)`` float32.  ``meta="f16"`` / ``"bf16"``: step
    and zero are rounded to binary16 / bfloat16 (still returned as float32
    values) and the codes are taken against the rounded grid.  ``axis="tokens"``: groups run
    along the second-to-last axis instead (per channel, ``group``
    consecutive tokens; the last group may be shorter): step/zero then have
    shape ``x.shape[:-2] + (ceil(N/group), d)``.
    """
    mk = META[meta]
    if axis == "tokens":
        return _quantize_tokens(np.ascontiguousarray(x), bits, group, mk)
    if axis != "dim":
        raise ValueError("axis must be 'dim' or 'tokens'")
    x = np.ascontiguousarray(x)
    d = x.shape[-1]
    rows = x.size // d if d else 0
    codes = np.zeros(x.shape[:-1] + (d * bits // 8,), np.uint8)
    step = np.zeros(x.shape[:-1] + (d // group,), np.float32)
    zero = np.zeros_like(step)
    if x.dtype == np.float32:
        rc = lib().kvo_quantize_f32_meta(_p(x), rows, d, group, bits, mk, _p(codes), _p(step), _p(zero))
    elif x.dtype == np.uint16:
        rc = lib().kvo_quantize_bf16_meta(_p(x), rows, d, group, bits, mk, _p(codes), _p(step), _p(zero))
    else:
        raise TypeError("x must be float32 or uint16 (bf16 bits)")
    _check(rc, "quantize")
    return codes, step, zero


def _quantize_tokens(x: np.ndarray, bits: int, group: int, mk: int):
    n, d = x.shape[-2], x.shape[-1]
    outer = x.size // (n * d) if n * d else 0
    ngr = (n + group - 1) // group
    codes = np.zeros(x.shape[:-1] + (d * bits // 8,), np.uint8)
    step = np.zeros(x.shape[:-2] + (ngr, d), np.float32)
    zero = np.zeros_like(step)
    if x.dtype == np.float32:
        f = lib().kvo_quantize_tokens_f32_meta
    elif x.dtype == np.uint16:
        f = lib().kvo_quantize_tokens_bf16_meta
    else:
        raise TypeError("x must be float32 or uint16 (bf16 bits)")
    _check(f(_p(x), outer, n, d, group, bits, mk, _p(codes), _p(step), _p(zero)), "quantize_tokens")
    return codes, step, zero


def round_fp16(x: float) -> float:
    return lib().kvo_round_fp16(float(x))


def round_bf16(x: float) -> float:
    return lib().kvo_round_bf16(float(x))


def unpack(codes: np.ndarray, d: int, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rows = codes.size // (d * bits // 8)
    out = np.zeros(codes.shape[:-1] + (d,), np.uint8)
    _check(lib().kvo_unpack(_p(codes), rows, d, bits, _p(out)), "unpack")
    return out


def pack(c: np.ndarray, bits: int) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    d = c.shape[-1]
    out = np.zeros(c.shape[:-1] + (d * bits // 8,), np.uint8)
    _check(lib().kvo_pack(_p(c), c.size // d, d, bits, _p(out)), "pack")
    return out


def dequant(codes, step, zero, d: int, group: int, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    step = np.ascontiguousarray(step, dtype=np.float32)
    zero = np.ascontiguousarray(zero, dtype=np.float32)
    rows = codes.size // (d * bits // 8)
    out = np.zeros(codes.shape[:-1] + (d,), np.float64)
    _check(lib().kvo_dequant(_p(codes), _p(step), _p(zero), rows, d, group, bits, _p(out)), "dequant")
    return out


# --------------------------------------------------------------------------
# Jensen bias
# --------------------------------------------------------------------------

def logsinhc(x: float) -> float:
    return lib().kvo_logsinhc(float(x))


def bias(q: np.ndarray, step: np.ndarray, group: int, tau: float, mode: str) -> float:
    """b for one query vector ``q`` (d,) and one cached key's ``step`` (d/group,)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    step = np.ascontiguousarray(step, dtype=np.float32)
    f = lib().kvo_bias_taylor if mode == "taylor" else lib().kvo_bias_exact
    return f(_p(q), _p(step), q.shape[0], group, float(tau))


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

class _Attn(C.Structure):
    _fields_ = [
        ("B", C.c_int64), ("Hq", C.c_int64), ("Hkv", C.c_int64), ("Nq", C.c_int64),
        ("Ncur", C.c_int64), ("Nc", C.c_int64), ("d", C.c_int32), ("group", C.c_int32),
        ("q", C.c_void_p), ("k_cur", C.c_void_p), ("v_cur", C.c_void_p),
        ("kc_codes", C.c_void_p), ("kc_step", C.c_void_p), ("kc_zero", C.c_void_p),
        ("vc_codes", C.c_void_p), ("vc_step", C.c_void_p), ("vc_zero", C.c_void_p),
        ("kbits", C.c_int32), ("vbits", C.c_int32), ("cap", C.c_int64),
        ("scale", C.c_double), ("corr", C.c_int32), ("causal", C.c_int32),
        ("kaxis", C.c_int32), ("vaxis", C.c_int32),
    ]


AXIS = {"dim": 0, "tokens": 1}


class Problem:
    """One attention problem in the library's layouts (host numpy arrays).

    q: uint16 bf16 bits [B][Hq][Nq][d]; k_cur, v_cur: uint16 [B][Hkv][Ncur][d];
    kcache/vcache: (codes, step, zero) with shapes [B][Hkv][cap][...]; with
    kaxis/vaxis "tokens" that cache's step and zero are
    [B][Hkv][ceil(cap/group)][d] (groups along the tokens).
    """

    def __init__(self, q, k_cur, v_cur, kcache, vcache, nc: int, kbits: int, vbits: int,
                 group: int, scale: float = 0.0, corr: str = "taylor", causal: bool = False,
                 kaxis: str = "dim", vaxis: str = "dim"):
        self.q = np.ascontiguousarray(q, dtype=np.uint16)
        B, Hq, Nq, d = self.q.shape
        self.k_cur = np.ascontiguousarray(k_cur, dtype=np.uint16)
        self.v_cur = np.ascontiguousarray(v_cur, dtype=np.uint16)
        Hkv, Ncur = self.k_cur.shape[1], self.k_cur.shape[2]
        self.kc = tuple(np.ascontiguousarray(a) for a in kcache)
        self.vc = tuple(np.ascontiguousarray(a) for a in vcache)
        cap = self.kc[0].shape[2] if nc > 0 else 0
        self.s = _Attn(B, Hq, Hkv, Nq, Ncur, nc, d, group,
                       _p(self.q).value, _p(self.k_cur).value, _p(self.v_cur).value,
                       _p(self.kc[0]).value, _p(self.kc[1]).value, _p(self.kc[2]).value,
                       _p(self.vc[0]).value, _p(self.vc[1]).value, _p(self.vc[2]).value,
                       kbits, vbits, cap, float(scale), CORR[corr], 1 if causal else 0,
                       AXIS[kaxis], AXIS[vaxis])
        self.shape = (B, Hq, Nq, d)

    def with_corr(self, corr: str) -> "Problem":
        self.s.corr = CORR[corr]
        return self

    def rows_total(self) -> int:
        B, Hq, Nq, _ = self.shape
        return B * Hq * Nq

    def attention(self, rows=None, threads: int = 0) -> np.ndarray:
        d = self.shape[3]
        if rows is None:
            n = self.rows_total()
            out = np.zeros((n, d), np.float64)
            rc = lib().kvo_attention(C.byref(self.s), None, n, _p(out), threads)
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            out = np.zeros((rows.size, d), np.float64)
            rc = lib().kvo_attention(C.byref(self.s), _p(rows), rows.size, _p(out), threads)
        _check(rc, "attention")
        return out

    def logits(self, row: int) -> np.ndarray:
        out = np.zeros(self.s.Nc + self.s.Ncur, np.float64)
        _check(lib().kvo_logits(C.byref(self.s), int(row), _p(out)), "logits")
        return out

    def attention_online(self, row: int, tile: int, bounds, cur_first: bool = False) -> np.ndarray:
        bounds = np.ascontiguousarray(bounds, dtype=np.int64)
        out = np.zeros(self.shape[3], np.float64)
        rc = lib().kvo_attention_online(C.byref(self.s), int(row), int(tile), _p(bounds),
                                        bounds.size - 1, int(cur_first), _p(out))
        _check(rc, "attention_online")
        return out

    def diagnostics(self, k_ref, rows=None, threads: int = 0):
        """Attention-balance statistics per row (kvo_diagnostics in the C
        source): ``stats`` [n][5] = lse_ref, lse_q, mass_ref, mass_q, kl and
        ``top`` [n][2][5] = top-5 key indices of the reference and of the
        quantised softmax (-1 past the visible keys).  ``k_ref``: uint16 bf16
        bits [B][Hkv][Nc][d], the cached keys before quantisation."""
        k_ref = np.ascontiguousarray(k_ref, dtype=np.uint16)
        if rows is None:
            n = self.rows_total()
            rp = None
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            n = rows.size
            rp = _p(rows)
        stats = np.zeros((n, 5), np.float64)
        top = np.zeros((n, 2, 5), np.int64)
        _check(lib().kvo_diagnostics(C.byref(self.s), _p(k_ref), rp, n, _p(stats), _p(top), threads),
               "diagnostics")
        return stats, top
