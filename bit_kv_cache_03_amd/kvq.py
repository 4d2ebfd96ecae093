"""ctypes binding of libkvq.so (declared in include/kvq.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  torch is used for device memory (tensors) and
streams.  Importing this module loads the library and raises ImportError if
it has not been built (``python -m bit_kv_cache_03_amd.build``); there is no
fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

(KV_OK, KV_ERR_NULL, KV_ERR_SHAPE, KV_ERR_UNSUPPORTED, KV_ERR_WORKSPACE, KV_ERR_ALIGN, KV_ERR_ALIAS, KV_ERR_HIP,
 KV_ERR_SCRATCH) = range(9)
STATIC_SCRATCH_BYTES = 64 << 20  # KV_STATIC_SCRATCH_BYTES
KV_BF16, KV_F32 = 0, 1
CORR = {"off": 0, "taylor": 1, "exact": 2}
PATH = {"auto": 0, "long": 1, "short": 2}

EXPORTED = ("kv_quantize", "kv_attention_workspace_size", "kv_attention_corrected",
            "kv_attention_corrected_static", "kv_attention_diagnostics", "kv_status_string", "kv_version")


class QTensor(C.Structure):
    """kv_qtensor."""
    _fields_ = [("codes", C.c_void_p), ("scale", C.c_void_p), ("zero", C.c_void_p),
                ("bits", C.c_int32), ("group", C.c_int32), ("cap", C.c_int64),
                ("page_table", C.c_void_p), ("page_size", C.c_int32), ("num_pages", C.c_int32),
                ("meta", C.c_int32), ("axis", C.c_int32), ("bound", C.c_void_p)]


META = {"f32": 0, "f16": 1, "bf16": 2}  # kv_meta: storage type of a cache tensor's step and zero point
AXIS = {"dim": 0, "tokens": 1}  # kv_axis: groups along the head dimension or along the tokens


class AttnArgs(C.Structure):
    """kv_attn_args."""
    _fields_ = [("B", C.c_int64), ("Hq", C.c_int64), ("Hkv", C.c_int64), ("Nq", C.c_int64),
                ("Ncur", C.c_int64), ("Nc", C.c_int64), ("d", C.c_int32),
                ("q", C.c_void_p), ("k_cur", C.c_void_p), ("v_cur", C.c_void_p),
                ("k_cache", C.POINTER(QTensor)), ("v_cache", C.POINTER(QTensor)),
                ("out", C.c_void_p), ("softmax_scale", C.c_float), ("corr", C.c_int32),
                ("path", C.c_int32), ("splits", C.c_int32), ("causal", C.c_int32),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
                ("append", C.c_int32), ("reserved", C.c_int32)]


class DiagArgs(C.Structure):
    """kv_diag_args."""
    _fields_ = [("B", C.c_int64), ("Hq", C.c_int64), ("Hkv", C.c_int64), ("Nq", C.c_int64),
                ("Ncur", C.c_int64), ("Nc", C.c_int64), ("d", C.c_int32), ("corr", C.c_int32),
                ("q", C.c_void_p), ("k_cur", C.c_void_p), ("k_ref", C.c_void_p),
                ("k_cache", C.POINTER(QTensor)), ("softmax_scale", C.c_float), ("causal", C.c_int32),
                ("out", C.c_void_p)]


DIAG_ROW_WORDS = 16  # kv_diag_row: 5 floats, 2 x 5 int32 indices, 1 reserved int32


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m bit_kv_cache_03_amd.build`")
    L = C.CDLL(LIB_PATH)
    L.kv_quantize.argtypes = [C.c_void_p, C.c_int, C.c_int64, C.c_int64, C.c_int64, C.c_int32,
                              C.POINTER(QTensor), C.c_int64, C.c_void_p]
    L.kv_quantize.restype = C.c_int
    L.kv_attention_workspace_size.argtypes = [C.POINTER(AttnArgs)]
    L.kv_attention_workspace_size.restype = C.c_size_t
    L.kv_attention_corrected.argtypes = [C.POINTER(AttnArgs), C.c_void_p]
    L.kv_attention_corrected.restype = C.c_int
    L.kv_attention_corrected_static.argtypes = [C.POINTER(AttnArgs), C.c_void_p]
    L.kv_attention_corrected_static.restype = C.c_int
    L.kv_attention_diagnostics.argtypes = [C.POINTER(DiagArgs), C.c_void_p]
    L.kv_attention_diagnostics.restype = C.c_int
    L.kv_status_string.argtypes = [C.c_int]
    L.kv_status_string.restype = C.c_char_p
    L.kv_version.restype = C.c_int32
    return L


lib = _load()


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib.kv_status_string(status).decode()} (status {status})")


def _check(status: int, what: str):
    if status != KV_OK:
        raise KvqError(status, what)


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _keep_for(t, stream) -> None:
    """A tensor allocated here from the current stream's pool but used by work
    enqueued on another `stream`: tell the caching allocator, so that its
    memory is not handed out again before that work has finished."""
    import torch
    if stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)


class QCache:
    """A quantized cache tensor (K or V): codes, step and zero-point on the GPU.

    Contiguous: [B][H][cap][...].  Paged (``page_table`` given: an int32 GPU
    tensor [B][cap // page_size] of page indices): pools of ``num_pages``
    pages [num_pages][H][page_size][...]; token t of (b, h) lives in page
    page_table[b][t // page_size] at row t % page_size.  ``meta``: "f32",
    "f16" (binary16 step and zero point) or "bf16" (bfloat16).  ``axis``: "dim" (groups of
    ``group`` channels per token) or "tokens" (per channel, groups of
    ``group`` tokens: step and zero [B][H][cap // group][d], paged
    [num_pages][H][page_size // group][d]).  ``bound``: keep the running
    bound of |dequantised value| per (b, h) that the quantiser raises and
    the attention reads instead of scanning the metadata (call
    ``reset_bound`` before refilling the cache from scratch)."""

    def __init__(self, B: int, H: int, cap: int, d: int, bits: int, group: int = 64, device="cuda",
                 page_table=None, page_size: int = 0, num_pages: int = 0, meta: str = "f32", axis: str = "dim",
                 bound: bool = True):
        import torch
        if meta not in META:
            raise ValueError(f"meta must be one of {sorted(META)}")
        if axis not in AXIS:
            raise ValueError(f"axis must be one of {sorted(AXIS)}")
        self.B, self.H, self.cap, self.d, self.bits, self.group = B, H, cap, d, bits, group
        self.page_table, self.page_size, self.num_pages = page_table, page_size, num_pages
        self.meta, self.axis = meta, axis
        lead = (num_pages, H, page_size) if page_table is not None else (B, H, cap)
        mdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[meta]
        self.codes = torch.zeros(lead + (d * bits // 8,), dtype=torch.uint8, device=device)
        mshape = lead[:2] + (lead[2] // group, d) if axis == "tokens" else lead + (d // group,)
        self.scale = torch.zeros(mshape, dtype=mdt, device=device)
        self.zero = torch.zeros(mshape, dtype=mdt, device=device)
        # running bound of |dequantised value| per (b, h), raised by every quantise
        self.bound = torch.zeros((B, H), dtype=torch.float32, device=device) if bound else None

    def reset_bound(self) -> None:
        if self.bound is not None:
            self.bound.zero_()

    def descriptor(self) -> QTensor:
        return QTensor(self.codes.data_ptr(), self.scale.data_ptr(), self.zero.data_ptr(),
                       self.bits, self.group, self.cap,
                       self.page_table.data_ptr() if self.page_table is not None else None,
                       self.page_size, self.num_pages, META[self.meta], AXIS[self.axis],
                       self.bound.data_ptr() if self.bound is not None else None)

    def logical(self, nc: int):
        """(codes, step, zero) of tokens [0, nc) in the contiguous [B][H][nc][...]
        order (a gather through the page table when paged); with axis
        "tokens", step and zero of the ceil(nc / group) token groups."""
        ng = -(-nc // self.group) if self.axis == "tokens" else nc
        if self.page_table is None:
            return self.codes[:, :, :nc], self.scale[:, :, :ng], self.zero[:, :, :ng]
        import torch

        def gather(x, n, per_row):  # per_row: tokens per stored row (1, or group)
            t = torch.arange(n, device=x.device) * per_row
            page = self.page_table.long()[:, t // self.page_size]  # [B][n]
            row = (t % self.page_size) // per_row
            return x[page, :, row.expand_as(page)].permute(0, 2, 1, 3)
        mper = self.group if self.axis == "tokens" else 1
        return gather(self.codes, nc, 1), gather(self.scale, ng, mper), gather(self.zero, ng, mper)


def quantize(x, cache: QCache, tok_offset: int = 0, stream=None) -> None:
    """Quantize x [B][H][N][d] (bf16 or fp32, on the GPU) into cache rows
    [tok_offset, tok_offset + N)."""
    import torch
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    xdt = {torch.bfloat16: KV_BF16, torch.float32: KV_F32}.get(x.dtype)
    if xdt is None:
        raise TypeError("x must be bfloat16 or float32")
    B, H, N, d = x.shape
    desc = cache.descriptor()
    _check(lib.kv_quantize(x.data_ptr(), xdt, B, H, N, d, C.byref(desc), tok_offset, _stream(stream)),
           "kv_quantize")


def make_args(q, k_cur, v_cur, k_cache: Optional[QCache], v_cache: Optional[QCache], nc: int, out,
              corr: str = "taylor", scale: float = 0.0, path: str = "auto", splits: int = 0,
              workspace=None, causal: bool = False, append: bool = False):
    """Fill kv_attn_args (keeps the descriptors alive on the returned object)."""
    B, Hq, Nq, d = q.shape
    Hkv = k_cur.shape[1] if k_cur is not None else k_cache.H
    ncur = k_cur.shape[2] if k_cur is not None else 0
    a = AttnArgs()
    a.B, a.Hq, a.Hkv, a.Nq, a.Ncur, a.Nc, a.d = B, Hq, Hkv, Nq, ncur, nc, d
    a.q, a.k_cur, a.v_cur, a.out = _ptr(q), _ptr(k_cur), _ptr(v_cur), _ptr(out)
    a._kd = k_cache.descriptor() if k_cache is not None else None
    a._vd = v_cache.descriptor() if v_cache is not None else None
    a.k_cache = C.pointer(a._kd) if a._kd is not None else None
    a.v_cache = C.pointer(a._vd) if a._vd is not None else None
    a.softmax_scale, a.corr, a.path, a.splits = scale, CORR[corr], PATH[path], splits
    a.causal = 1 if causal else 0
    a.append = 1 if append else 0
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return a


def workspace_size(args: AttnArgs) -> int:
    return lib.kv_attention_workspace_size(C.byref(args))


def attention(q, k_cur, v_cur, k_cache: Optional[QCache], v_cache: Optional[QCache], nc: int,
              corr: str = "taylor", scale: float = 0.0, path: str = "auto", splits: int = 0,
              out=None, workspace=None, stream=None, causal: bool = False, append: bool = False):
    """Corrected attention of q [B][Hq][Nq][d] (bf16) over the first nc tokens
    of the quantized caches and the bf16 current chunk [B][Hkv][Ncur][d]
    (causal: end-aligned causal mask within the current chunk; append: the
    same call also quantises the chunk into cache rows [nc, nc + Ncur)).
    Returns out [B][Hq][Nq][d] bf16."""
    import torch
    if out is None:
        out = torch.empty_like(q)
        _keep_for(out, stream)
    args = make_args(q, k_cur, v_cur, k_cache, v_cache, nc, out, corr, scale, path, splits, workspace, causal,
                     append)
    need = workspace_size(args)
    if need > 0 and (workspace is None or args.workspace_bytes < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _keep_for(workspace, stream)
        args.workspace, args.workspace_bytes = workspace.data_ptr(), need
    _check(lib.kv_attention_corrected(C.byref(args), _stream(stream)), "kv_attention_corrected")
    return out


def make_diag_args(q, k_cur, k_ref, k_cache: Optional[QCache], nc: int, out, corr: str = "taylor",
                   scale: float = 0.0, causal: bool = False):
    """Fill kv_diag_args (keeps the descriptor alive on the returned object)."""
    B, Hq, Nq, d = q.shape
    Hkv = k_cur.shape[1] if k_cur is not None else k_cache.H
    ncur = k_cur.shape[2] if k_cur is not None else 0
    a = DiagArgs()
    a.B, a.Hq, a.Hkv, a.Nq, a.Ncur, a.Nc, a.d = B, Hq, Hkv, Nq, ncur, nc, d
    a.corr = CORR[corr]
    a.q, a.k_cur, a.k_ref = _ptr(q), _ptr(k_cur), _ptr(k_ref)
    a._kd = k_cache.descriptor() if k_cache is not None else None
    a.k_cache = C.pointer(a._kd) if a._kd is not None else None
    a.softmax_scale, a.causal = scale, 1 if causal else 0
    a.out = _ptr(out)
    return a


def diagnostics(q, k_cur, k_ref, k_cache: Optional[QCache], nc: int, corr: str = "taylor",
                scale: float = 0.0, causal: bool = False, out=None, stream=None):
    """Attention-balance statistics of every query row (kv_attention_diagnostics):
    the softmax over the unquantised cached keys k_ref [B][Hkv][nc][d] (bf16)
    against the one over the first nc tokens of the quantised k_cache (with
    `corr`), both with the bf16 current keys k_cur.  Returns an int32 tensor
    [B*Hq*Nq][16] of kv_diag_row records: columns 0..4 are the fp32 lse_ref,
    lse_q, mass_ref, mass_q, kl (``.view(torch.float32)``), 5..9 the
    reference top-5 key indices, 10..14 the quantised ones."""
    import torch
    B, Hq, Nq, _ = q.shape
    if out is None:
        out = torch.empty((B * Hq * Nq, DIAG_ROW_WORDS), dtype=torch.int32, device=q.device)
        _keep_for(out, stream)
    args = make_diag_args(q, k_cur, k_ref, k_cache, nc, out, corr, scale, causal)
    _check(lib.kv_attention_diagnostics(C.byref(args), _stream(stream)), "kv_attention_diagnostics")
    return out
