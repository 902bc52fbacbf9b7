"""Thin Python binding of libattn's C ABI (include/attn.h).

Only argument marshalling lives here: torch tensors supply device pointers, strides and
the current HIP stream; every step of the computation runs in libattn's HIP kernels.
There is no fallback: if libattn.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_F32, ATTN_BF16 = 0, 1
ATTN_OK, ATTN_ERR_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = 0, -1, -2, -3, -4

# The entry points include/attn.h declares (checked by the CPU test suite).
EXPORTS = ("attn_prep", "attn_prefill", "attn_prefill_chunk", "attn_prefill_chunk_paged", "attn_decode", "attn_decode_workspace_size",
           "attn_decode_default_splits", "attn_decode_paged", "attn_kv_quantize", "attn_decode_q",
           "attn_decode_q_paged", "attn_decode_q_default_splits", "attn_rows", "attn_rows8_layout", "attn_rows8_quantize",
           "attn_rows8_attend", "attn_rows8", "attn_row_norm_rope", "attn_key_bound", "attn_supported",
           "attn_status_str", "attn_last_error", "attn_decode_static", "attn_decode_static_scratch_bytes")


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (status %d)" % (message, status))
        self.status = status


class attn_headprep_t(ctypes.Structure):
    _fields_ = [("qw", ctypes.c_void_p), ("kw", ctypes.c_void_p), ("cos", ctypes.c_void_p),
                ("sin", ctypes.c_void_p), ("half", ctypes.c_int64), ("table_rows", ctypes.c_int64),
                ("eps", ctypes.c_double), ("pairs", ctypes.c_int64), ("kmax", ctypes.c_double)]


_lib = None
_i64, _vp, _dbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double


def load_library(path: str = LIB_PATH):
    """Load libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libattn.so is not built (expected at %s); run "
                          "`python -m transformer_attention_headprep_amd.build`" % path)
    lib = ctypes.CDLL(path)
    hp = ctypes.POINTER(attn_headprep_t)
    lib.attn_prep.argtypes = [_vp, _vp] + [_i64] * 8 + [hp, ctypes.c_int, _vp]
    lib.attn_prep.restype = ctypes.c_int
    lib.attn_prefill.argtypes = [_vp, _vp, _vp, _vp] + [_i64] * 10 + [hp, ctypes.c_int, _dbl,
                                                                         ctypes.c_int, _vp]
    lib.attn_prefill.restype = ctypes.c_int
    lib.attn_prefill_chunk.argtypes = [_vp] * 6 + [_i64] * 7 + [_vp, hp, ctypes.c_int, _dbl, ctypes.c_int, _vp]
    lib.attn_prefill_chunk.restype = ctypes.c_int
    lib.attn_prefill_chunk_paged.argtypes = [_vp] * 6 + [_i64] * 7 + [_vp, _i64, _i64, _vp, hp, ctypes.c_int, _dbl,
                                                                      ctypes.c_int, _vp]
    lib.attn_prefill_chunk_paged.restype = ctypes.c_int
    lib.attn_decode.argtypes = [_vp, _vp, _vp, _vp] + [_i64] * 5 + [_vp, _vp, _i64, _i64, hp, _dbl, _i64,
                                                                    _vp, ctypes.c_size_t,
                                                                    ctypes.c_int, _vp]
    lib.attn_decode.restype = ctypes.c_int
    lib.attn_decode_workspace_size.argtypes = [_i64] * 6
    lib.attn_decode_workspace_size.restype = ctypes.c_size_t
    lib.attn_decode_default_splits.argtypes = [_i64] * 5
    lib.attn_decode_default_splits.restype = _i64
    lib.attn_kv_quantize.argtypes = [_vp] + [_i64] * 6 + [_vp, _vp, _i64, _i64, ctypes.c_int, _vp]
    lib.attn_kv_quantize.restype = ctypes.c_int
    lib.attn_decode_q.argtypes = [_vp] * 6 + [_i64] * 7 + [_vp, _vp, _i64, _i64, hp, _dbl, _i64, _vp, ctypes.c_size_t,
                                                         ctypes.c_int, _vp]
    lib.attn_decode_q.restype = ctypes.c_int
    lib.attn_decode_q_default_splits.argtypes = [_i64] * 5
    lib.attn_decode_q_default_splits.restype = _i64
    lib.attn_rows8_layout.argtypes = [_i64] * 5 + [_vp]
    lib.attn_rows8_layout.restype = ctypes.c_size_t
    lib.attn_rows8_quantize.argtypes = [_vp] + [_i64] * 5 + [hp, _vp, ctypes.c_size_t, _vp]
    lib.attn_rows8_quantize.restype = ctypes.c_int
    lib.attn_rows8_attend.argtypes = [_vp, ctypes.c_size_t] + [_i64] * 5 + [_vp, _vp]
    lib.attn_rows8_attend.restype = ctypes.c_int
    lib.attn_rows8.argtypes = [_vp] + [_i64] * 5 + [_vp, hp, _vp, ctypes.c_size_t, _vp]
    lib.attn_rows8.restype = ctypes.c_int
    lib.attn_rows.argtypes = [_vp] + [_i64] * 5 + [_vp, hp, ctypes.c_int, _vp]
    lib.attn_rows.restype = ctypes.c_int
    lib.attn_row_norm_rope.argtypes = [_vp] + [_i64] * 4 + [_vp, _vp, _vp, _dbl, ctypes.c_int, _vp]
    lib.attn_row_norm_rope.restype = ctypes.c_int
    lib.attn_decode_paged.argtypes = [_vp, _vp, _vp, _vp] + [_i64] * 6 + [_vp, _i64, _vp, _vp, _i64, _i64, hp, _dbl, _i64,
                                                                            _vp, ctypes.c_size_t, ctypes.c_int, _vp]
    lib.attn_decode_paged.restype = ctypes.c_int
    lib.attn_decode_static.argtypes = [_vp, _vp, _vp, _vp] + [_i64] * 5 + [_vp, _vp, _i64, _i64, hp, _dbl, _i64,
                                                                           ctypes.c_int, _vp]
    lib.attn_decode_static.restype = ctypes.c_int
    lib.attn_decode_static_scratch_bytes.argtypes = []
    lib.attn_decode_static_scratch_bytes.restype = ctypes.c_size_t
    lib.attn_decode_q_paged.argtypes = [_vp] * 6 + [_i64] * 8 + [_vp, _i64, _vp, _vp, _i64, _i64, hp, _dbl, _i64, _vp,
                                                                  ctypes.c_size_t, ctypes.c_int, _vp]
    lib.attn_decode_q_paged.restype = ctypes.c_int
    lib.attn_key_bound.argtypes = [_vp, _i64]
    lib.attn_key_bound.restype = _dbl
    lib.attn_supported.argtypes = [_i64, ctypes.c_int]
    lib.attn_supported.restype = ctypes.c_int
    lib.attn_status_str.argtypes = [ctypes.c_int]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != ATTN_OK:
        lib = load_library()
        raise AttnError(status, (lib.attn_last_error() or b"").decode() or
                        lib.attn_status_str(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _row_stride(t: torch.Tensor, name: str) -> int:
    """[B, S, H, D] view whose rows are `stride(1)` elements apart (heads contiguous)."""
    if t.dim() != 4:
        raise ValueError("%s must be [batch, seq, heads, d]" % name)
    B, S, H, D = t.shape
    if t.stride(3) != 1 or (H > 1 and t.stride(2) != D):
        raise ValueError("%s: heads and values must be contiguous inside a row" % name)
    if B > 1 and t.stride(0) != S * t.stride(1):
        raise ValueError("%s: sequences must follow each other (batch stride = seq * row stride)" % name)
    return t.stride(1) if S > 1 else (t.stride(0) if B > 1 else H * D)


@dataclass
class HeadPrep:
    """The HeadPrep record {qw, kw, cos, sin, eps} as device f32 tensors; pairs=True turns
    adjacent values (2i, 2i + 1) rather than split halves (i, i + half).  kmax > 0 is the
    caller's bound on the norm of every key row the attention reads (see attn_headprep_t;
    key_bound() gives the one HeadPrep with weights kw guarantees)."""
    qw: torch.Tensor
    kw: torch.Tensor
    cos: torch.Tensor | None
    sin: torch.Tensor | None
    eps: float
    pairs: bool = False
    kmax: float = 0.0

    @property
    def half(self) -> int:
        return 0 if self.cos is None else int(self.cos.shape[1])

    @property
    def table_rows(self) -> int:
        return 0 if self.cos is None else int(self.cos.shape[0])

    def struct(self) -> attn_headprep_t:
        for name in ("qw", "kw", "cos", "sin"):
            t = getattr(self, name)
            if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
                raise ValueError("HeadPrep.%s must be a contiguous float32 tensor" % name)
        half = self.half
        return attn_headprep_t(
            self.qw.data_ptr() if self.qw is not None else None,
            self.kw.data_ptr() if self.kw is not None else None,
            self.cos.data_ptr() if half else None, self.sin.data_ptr() if half else None,
            half, int(self.cos.shape[0]) if half else 0, float(self.eps), int(bool(self.pairs)),
            float(self.kmax))


def key_bound(kw, d: int) -> float:
    """attn_key_bound: the bound HeadPrep with weights kw (host array or tensor of d
    values) guarantees on the norm of every key row it writes, for HeadPrep.kmax."""
    if isinstance(kw, torch.Tensor):
        kw = kw.detach().to("cpu", torch.float32).contiguous()
    else:
        kw = torch.as_tensor(kw, dtype=torch.float32).contiguous()
    if kw.numel() != d:
        raise ValueError("kw must hold d = %d values" % d)
    lib = load_library()
    return float(lib.attn_key_bound(ctypes.c_void_p(kw.data_ptr()), ctypes.c_int64(d)))


def attn_supported(d: int, dtype: torch.dtype) -> bool:
    return bool(load_library().attn_supported(d, ATTN_BF16 if dtype == torch.bfloat16 else ATTN_F32))


def attn_prep(q, k, prep: HeadPrep, pos0: int = 0, stream=None) -> None:
    """HeadPrep in place on q [B, S, Hq, D] and/or k [B, S, Hkv, D]."""
    lib = load_library()
    ref = q if q is not None else k
    B, S = ref.shape[0], ref.shape[1]
    D = ref.shape[3]
    hq = q.shape[2] if q is not None else 0
    hkv = k.shape[2] if k is not None else 0
    qrs = _row_stride(q, "q") if q is not None else 0
    krs = _row_stride(k, "k") if k is not None else 0
    if q is not None and k is not None and q.dtype != k.dtype:
        raise TypeError("q and k must share a dtype")
    st = prep.struct()
    _check(lib.attn_prep(_ptr(q), _ptr(k), B, S, hq, hkv, D, qrs, krs, pos0, ctypes.byref(st),
                         _dtype_code(ref), _stream(stream)))


def attn_prefill(q, k, v, out=None, prep: HeadPrep | None = None, pos0: int = 0,
                 causal: bool = True, scale: float | None = None, stream=None) -> torch.Tensor:
    """out = softmax(prep(q) prep(k)^T scale [+ causal]) v; with prep, k is prepped in place."""
    lib = load_library()
    B, S, hq, D = q.shape
    hkv = k.shape[2]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if not (q.dtype == k.dtype == v.dtype == out.dtype):
        raise TypeError("q, k, v and out must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = prep.struct() if prep is not None else None
    _check(lib.attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, S, hq, hkv, D,
                            _row_stride(q, "q"), _row_stride(k, "k"), _row_stride(v, "v"),
                            _row_stride(out, "out"), pos0,
                            ctypes.byref(st) if st is not None else None, int(bool(causal)),
                            float(scale), _dtype_code(q), _stream(stream)))
    return out


def _past(past, B):
    if past is None:
        return None
    if past.dtype != torch.int32 or past.dim() != 1 or past.shape[0] != B or not past.is_contiguous():
        raise TypeError("past must be a contiguous int32 [B] device tensor")
    return _ptr(past)


def attn_prefill_chunk(q, k_new, v_new, k_cache, v_cache, n_past: int, out=None,
                       prep: HeadPrep | None = None, causal: bool = True, scale: float | None = None,
                       stream=None, past=None) -> torch.Tensor:
    """A chunk q [B, tq, Hq, D] against caches [B, capacity, Hkv, D] holding n_past rows:
    appends prep(k_new) and v_new at rows n_past .., then attends rows 0 .. n_past + tq - 1.
    With ``past`` (int32 [B] on the device) sequence b holds past[b] rows instead, and
    n_past is the bound on every past[b]."""
    lib = load_library()
    B, tq, hq, D = q.shape
    cap, hkv = k_cache.shape[1], k_cache.shape[2]
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.dtype != q.dtype:
            raise TypeError("all operands must share a dtype")
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = prep.struct() if prep is not None else None
    _check(lib.attn_prefill_chunk(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                  B, tq, hq, hkv, D, cap, n_past, _past(past, B),
                                  ctypes.byref(st) if st is not None else None, int(bool(causal)),
                                  float(scale), _dtype_code(q), _stream(stream)))
    return out


def attn_prefill_chunk_paged(q, k_new, v_new, k_pool, v_pool, pages, n_past: int, out=None,
                             prep: HeadPrep | None = None, causal: bool = True, scale: float | None = None,
                             stream=None, past=None) -> torch.Tensor:
    """attn_prefill_chunk with the cache in a paged pool k_pool, v_pool [num_pages, page_rows,
    Hkv, D]; pages [B, max_pages] int32 maps each sequence's rows to pages."""
    lib = load_library()
    B, tq, hq, D = q.shape
    num_pages, page_rows, hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_pool", k_pool), ("v_pool", v_pool)):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.dtype != q.dtype:
            raise TypeError("all operands must share a dtype")
    if pages.dtype != torch.int32 or pages.dim() != 2 or pages.shape[0] != B or not pages.is_contiguous():
        raise TypeError("pages must be a contiguous int32 [B, max_pages] device tensor")
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = prep.struct() if prep is not None else None
    _check(lib.attn_prefill_chunk_paged(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(out),
                                        B, tq, hq, hkv, D, num_pages, page_rows, _ptr(pages), pages.shape[1], n_past,
                                        _past(past, B), ctypes.byref(st) if st is not None else None, int(bool(causal)),
                                        float(scale), _dtype_code(q), _stream(stream)))
    return out


@dataclass
class QuantCache:
    """A quantised KV cache of one tensor (K or V): codes uint8 [B, hkv, capacity, d bits / 8]
    and params f32 [B, hkv, capacity, 2] (lo, step) on the device."""
    codes: torch.Tensor
    params: torch.Tensor
    bits: int

    @staticmethod
    def empty(batch: int, heads: int, capacity: int, d: int, bits: int, device="cuda") -> "QuantCache":
        return QuantCache(torch.zeros(batch, heads, capacity, d * bits // 8, dtype=torch.uint8, device=device),
                          torch.zeros(batch, heads, capacity, 2, dtype=torch.float32, device=device), bits)

    @property
    def capacity(self) -> int:
        return int(self.codes.shape[2])


def attn_kv_quantize(x, cache: QuantCache, row0: int = 0, stream=None) -> None:
    """Code x [B, S, H, D] (bf16 or f32) into cache rows row0 .. row0 + S - 1."""
    lib = load_library()
    B, S, H, D = x.shape
    for t in (cache.codes, cache.params):
        if not t.is_contiguous():
            raise ValueError("the cache tensors must be contiguous")
    if tuple(cache.codes.shape) != (B, H, cache.capacity, D * cache.bits // 8):
        raise ValueError("cache codes must be [B, H, capacity, D * bits / 8]")
    _check(lib.attn_kv_quantize(_ptr(x), B, S, H, D, _row_stride(x, "x"), cache.bits, _ptr(cache.codes),
                                _ptr(cache.params), cache.capacity, row0, _dtype_code(x), _stream(stream)))


def attn_decode_q(q, k: QuantCache, v: QuantCache, lens, pos, max_len: int, prep: HeadPrep | None = None,
                  scale: float | None = None, splits: int = 0, workspace=None, out=None, stream=None,
                  max_pos: int | None = None) -> torch.Tensor:
    """One bf16 query row per sequence (q [B, Hq, D]) against quantised caches."""
    lib = load_library()
    B, hq, D = q.shape
    hkv, cap = k.codes.shape[1], k.capacity
    if q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bfloat16 tensor")
    if lens.dtype != torch.int32 or (pos is not None and pos.dtype != torch.int32):
        raise TypeError("lens and pos must be int32 device tensors")
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if splits == 0:
        splits = int(lib.attn_decode_q_default_splits(B, hq, hkv, max_len, k.bits))
    need = decode_workspace_size(B, hq, hkv, D, max_len, splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = prep.struct() if prep is not None else None
    _check(lib.attn_decode_q(_ptr(q), _ptr(k.codes), _ptr(k.params), _ptr(v.codes), _ptr(v.params), _ptr(out),
                             B, hq, hkv, D, cap, k.bits, v.bits, _ptr(lens), _ptr(pos), max_len,
                             _max_pos(prep, max_pos), ctypes.byref(st) if st is not None else None, float(scale), splits, _ptr(workspace),
                             0 if workspace is None else workspace.numel() * workspace.element_size(),
                             ATTN_BF16, _stream(stream)))
    return out


def attn_decode_q_paged(q, k: QuantCache, v: QuantCache, pages, lens, pos, max_len: int,
                        prep: HeadPrep | None = None, scale: float | None = None, splits: int = 0, workspace=None,
                        out=None, stream=None, max_pos: int | None = None) -> torch.Tensor:
    """attn_decode_q over a paged pool: k and v are QuantCaches whose batch axis is the pool's
    pages (capacity = page_rows); pages [B, max_pages] int32 maps sequence rows to pages."""
    lib = load_library()
    B, hq, D = q.shape
    num_pages, hkv, page_rows = k.codes.shape[0], k.codes.shape[1], k.capacity
    if q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bfloat16 tensor")
    if pages.dtype != torch.int32 or pages.dim() != 2 or pages.shape[0] != B or not pages.is_contiguous():
        raise TypeError("pages must be a contiguous int32 [B, max_pages] device tensor")
    if lens.dtype != torch.int32 or (pos is not None and pos.dtype != torch.int32):
        raise TypeError("lens and pos must be int32 device tensors")
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if splits == 0:
        splits = int(lib.attn_decode_q_default_splits(B, hq, hkv, max_len, k.bits))
    need = decode_workspace_size(B, hq, hkv, D, max_len, splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = prep.struct() if prep is not None else None
    _check(lib.attn_decode_q_paged(_ptr(q), _ptr(k.codes), _ptr(k.params), _ptr(v.codes), _ptr(v.params), _ptr(out),
                                   B, hq, hkv, D, num_pages, page_rows, k.bits, v.bits, _ptr(pages), pages.shape[1],
                                   _ptr(lens), _ptr(pos), max_len, _max_pos(prep, max_pos),
                                   ctypes.byref(st) if st is not None else None,
                                   float(scale), splits, _ptr(workspace),
                                   0 if workspace is None else workspace.numel() * workspace.element_size(),
                                   ATTN_BF16, _stream(stream)))
    return out


def attn_rows(qkv, heads: int, head: int, group: int = 0, queries: int = 0, out=None,
              prep: HeadPrep | None = None, stream=None) -> torch.Tensor:
    """Full attention of packed rows qkv [n, 3 * heads * head] (q, k, v of every head), each
    query seeing the keys of its group of `group` rows (0: all); out [queries or n, heads * head].
    With prep, q and k are prepped in place in qkv first (row r at table row r)."""
    lib = load_library()
    if qkv.dim() != 2 or not qkv.is_contiguous() or qkv.shape[1] != 3 * heads * head:
        raise ValueError("qkv must be a contiguous [n, 3 * heads * head] tensor")
    n = qkv.shape[0]
    nq = queries if queries else n
    if out is None:
        out = torch.empty(nq, heads * head, dtype=qkv.dtype, device=qkv.device)
    if out.dtype != qkv.dtype or not out.is_contiguous() or tuple(out.shape) != (nq, heads * head):
        raise ValueError("out must be a contiguous [queries or n, heads * head] tensor of qkv's dtype")
    st = prep.struct() if prep is not None else None
    _check(lib.attn_rows(_ptr(qkv), n, heads, head, group, queries, _ptr(out),
                         ctypes.byref(st) if st is not None else None, _dtype_code(qkv), _stream(stream)))
    return out


ROWS8_PARTS = ("q8", "sq", "k8", "sk", "v8t", "sv", "vmax")


def rows8_layout(n: int, heads: int, head: int, group: int = 0, queries: int = 0):
    """(workspace bytes, {part: byte offset}) of the quantised rows path's workspace."""
    offs = (ctypes.c_int64 * 7)()
    total = int(load_library().attn_rows8_layout(n, heads, head, group, queries, offs))
    if total == 0:
        raise ValueError("bad sizes for the quantised rows path")
    return total, dict(zip(ROWS8_PARTS, list(offs)))


def attn_rows8(qkv, heads: int, head: int, group: int = 0, queries: int = 0, out=None, prep: HeadPrep | None = None,
               workspace=None, stream=None) -> torch.Tensor:
    """attn_rows' quantised path: 8-bit operands (coded with HeadPrep in the quantizing pass,
    qkv untouched), Q K^T on INT8 and P V on E4M3; out [queries or n, heads * head] bf16."""
    lib = load_library()
    if qkv.dtype != torch.bfloat16 or qkv.dim() != 2 or not qkv.is_contiguous() or qkv.shape[1] != 3 * heads * head:
        raise ValueError("qkv must be a contiguous bf16 [n, 3 * heads * head] tensor")
    n = qkv.shape[0]
    nq = queries if queries else n
    if out is None:
        out = torch.empty(nq, heads * head, dtype=torch.bfloat16, device=qkv.device)
    total, _ = rows8_layout(n, heads, head, group, queries)
    if workspace is None:
        workspace = torch.empty(total, dtype=torch.uint8, device=qkv.device)
    st = prep.struct() if prep is not None else None
    _check(lib.attn_rows8(_ptr(qkv), n, heads, head, group, queries, _ptr(out),
                          ctypes.byref(st) if st is not None else None, _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def attn_rows8_quantize(qkv, heads: int, head: int, workspace, group: int = 0, queries: int = 0,
                        prep: HeadPrep | None = None, stream=None) -> None:
    lib = load_library()
    st = prep.struct() if prep is not None else None
    _check(lib.attn_rows8_quantize(_ptr(qkv), qkv.shape[0], heads, head, group, queries,
                                   ctypes.byref(st) if st is not None else None, _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


def attn_rows8_attend(workspace, n: int, heads: int, head: int, group: int = 0, queries: int = 0, out=None,
                      stream=None) -> torch.Tensor:
    lib = load_library()
    nq = queries if queries else n
    if out is None:
        out = torch.empty(nq, heads * head, dtype=torch.bfloat16, device=workspace.device)
    _check(lib.attn_rows8_attend(_ptr(workspace), workspace.numel() * workspace.element_size(), n, heads, head, group,
                                 queries, _ptr(out), _stream(stream)))
    return out


def attn_row_norm_rope(x, w, eps: float, cos=None, sin=None, head: int | None = None, stream=None) -> None:
    """In place on x [rows, width] (row-strided, values contiguous): whole-row RMS norm times w,
    then with cos/sin [rows, width / 2] each head of `head` values turned by split halves."""
    lib = load_library()
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [rows, width] with contiguous rows")
    rows, width = x.shape
    for name, t in (("w", w), ("cos", cos), ("sin", sin)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("%s must be a contiguous float32 tensor" % name)
    if cos is not None and tuple(cos.shape) != (rows, width // 2):
        raise ValueError("cos/sin must be [rows, width / 2]")
    if (cos is None) != (sin is None) or (sin is not None and sin.shape != cos.shape):
        raise ValueError("cos and sin go together, of one shape")
    if head is None:
        head = width
    rs = x.stride(0) if rows > 1 else width
    _check(lib.attn_row_norm_rope(_ptr(x), rows, width, head, rs, _ptr(w), _ptr(cos), _ptr(sin), float(eps),
                                  _dtype_code(x), _stream(stream)))


def decode_workspace_size(batch: int, hq: int, hkv: int, d: int, max_len: int, splits: int = 0) -> int:
    return int(load_library().attn_decode_workspace_size(batch, hq, hkv, d, max_len, splits))


def decode_q_default_splits(batch: int, hq: int, hkv: int, max_len: int, k_bits: int) -> int:
    return int(load_library().attn_decode_q_default_splits(batch, hq, hkv, max_len, k_bits))


def _max_pos(prep: "HeadPrep | None", max_pos: "int | None") -> int:
    """The host bound on every pos[b]: the caller's, else the last row of the tables."""
    if max_pos is not None:
        return int(max_pos)
    return prep.table_rows - 1 if prep is not None and prep.half else 0


def decode_default_splits(batch: int, hq: int, hkv: int, d: int, max_len: int) -> int:
    return int(load_library().attn_decode_default_splits(batch, hq, hkv, d, max_len))


def attn_decode(q, k_cache, v_cache, lens, pos, max_len: int, prep: HeadPrep | None = None,
                scale: float | None = None, splits: int = 0, workspace=None, out=None,
                stream=None, max_pos: int | None = None) -> torch.Tensor:
    """One query row per sequence (q [B, Hq, D]) against caches [B, capacity, Hkv, D]."""
    lib = load_library()
    B, hq, D = q.shape
    cap, hkv = k_cache.shape[1], k_cache.shape[2]
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if lens.dtype != torch.int32 or (pos is not None and pos.dtype != torch.int32):
        raise TypeError("lens and pos must be int32 device tensors")
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = decode_workspace_size(B, hq, hkv, D, max_len, splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = prep.struct() if prep is not None else None
    _check(lib.attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), B, hq, hkv, D, cap,
                           _ptr(lens), _ptr(pos), max_len, _max_pos(prep, max_pos),
                           ctypes.byref(st) if st is not None else None, float(scale), splits,
                           _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
                           _dtype_code(q), _stream(stream)))
    return out


def attn_decode_static(q, k_cache, v_cache, lens, pos, max_len: int, prep: HeadPrep | None = None,
                       scale: float | None = None, splits: int = 0, out=None, stream=None,
                       max_pos: int | None = None) -> torch.Tensor:
    """attn_decode with its split partials in the library's own device scratch (no
    workspace).  `out` should be given by callers that cannot allocate."""
    lib = load_library()
    B, hq, D = q.shape
    cap, hkv = k_cache.shape[1], k_cache.shape[2]
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if lens.dtype != torch.int32 or (pos is not None and pos.dtype != torch.int32):
        raise TypeError("lens and pos must be int32 device tensors")
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = prep.struct() if prep is not None else None
    _check(lib.attn_decode_static(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), B, hq, hkv, D, cap,
                                  _ptr(lens), _ptr(pos), max_len, _max_pos(prep, max_pos),
                                  ctypes.byref(st) if st is not None else None, float(scale), splits,
                                  _dtype_code(q), _stream(stream)))
    return out


def decode_static_scratch_bytes() -> int:
    """Bytes of the device scratch attn_decode_static uses."""
    return int(load_library().attn_decode_static_scratch_bytes())


def attn_decode_paged(q, k_pool, v_pool, pages, lens, pos, max_len: int, prep: HeadPrep | None = None,
                      scale: float | None = None, splits: int = 0, workspace=None, out=None,
                      stream=None, max_pos: int | None = None) -> torch.Tensor:
    """One bf16 query row per sequence (q [B, Hq, D]) against a paged pool k_pool, v_pool
    [num_pages, page_rows, Hkv, D]; pages [B, max_pages] int32 maps sequence rows to pages."""
    lib = load_library()
    B, hq, D = q.shape
    num_pages, page_rows, hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("pages", pages)):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if pages.dtype != torch.int32 or pages.dim() != 2 or pages.shape[0] != B:
        raise TypeError("pages must be an int32 [B, max_pages] device tensor")
    if lens.dtype != torch.int32 or (pos is not None and pos.dtype != torch.int32):
        raise TypeError("lens and pos must be int32 device tensors")
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = decode_workspace_size(B, hq, hkv, D, max_len, splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = prep.struct() if prep is not None else None
    _check(lib.attn_decode_paged(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out), B, hq, hkv, D, num_pages, page_rows,
                                 _ptr(pages), pages.shape[1], _ptr(lens), _ptr(pos), max_len,
                                 _max_pos(prep, max_pos), ctypes.byref(st) if st is not None else None, float(scale), splits,
                                 _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
                                 _dtype_code(q), _stream(stream)))
    return out
