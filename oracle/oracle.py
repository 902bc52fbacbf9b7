"""ctypes binding of the f64 oracle (``oracle.c``) plus the path's compositions (prefill,
chunked prefill against a cache, decode).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Inputs are numpy arrays of any
float dtype; they are widened to f64, which is exact for f32 and bf16 values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_int64)


def library_path() -> str:
    return _LIB


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (IEEE f64, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c99",
             "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"],
            check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # A planted-mistake copy of the oracle (built by the mutation test) can be
        # swapped in through this variable; by default the library built from oracle.c.
        path = os.environ.get("ATTN_ORACLE_LIB") or build()
        lib = ctypes.CDLL(path)
        lib.oracle_headprep.argtypes = [_dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64, _lp,
                                        ctypes.c_double]
        lib.oracle_headprep.restype = ctypes.c_int
        lib.oracle_headprep_pairs.argtypes = lib.oracle_headprep.argtypes
        lib.oracle_headprep_pairs.restype = ctypes.c_int
        lib.oracle_row_norm_rope.argtypes = [_dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _dp,
                                             _dp, _dp, ctypes.c_int64, _lp, ctypes.c_double]
        lib.oracle_row_norm_rope.restype = ctypes.c_int
        att = [_dp, _dp, _dp, _dp] + [ctypes.c_int64] * 7 + [ctypes.c_double, ctypes.c_int, _lp]
        lib.oracle_attention.argtypes = att
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention_rows.argtypes = att + [_lp, ctypes.c_int64]
        lib.oracle_attention_rows.restype = ctypes.c_int
        fp = ctypes.POINTER(ctypes.c_float)
        ip = ctypes.POINTER(ctypes.c_int32)
        lib.oracle_kv_quantize.argtypes = [fp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ip, fp, fp, ip]
        lib.oracle_kv_quantize.restype = ctypes.c_int
        i8p = ctypes.POINTER(ctypes.c_int8)
        lib.oracle_int8_code.argtypes = [fp, ctypes.c_int64, ctypes.c_int64, i8p, fp]
        lib.oracle_int8_code.restype = ctypes.c_int
        lib.oracle_e4m3_code.argtypes = [fp, ctypes.c_int64, ctypes.c_int64, fp, fp]
        lib.oracle_e4m3_code.restype = ctypes.c_int
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    return int(_load().oracle_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    if a is None:
        return None
    if a.dtype == np.float64:
        return a.ctypes.data_as(_dp)
    return a.ctypes.data_as(_lp)


def headprep(x, w, cos, sin, half: int, pos, eps: float, pairs: bool = False) -> np.ndarray:
    """HeadPrep of x [..., heads, d] (gizml:netops, Types > HeadPrep), returned as a new
    f64 array.  ``pos`` gives the table row of each leading index (shape x.shape[:-2]).
    pairs=False: value e < half turns with e + half (split halves); pairs=True: value 2i
    with 2i + 1 (FLUX.3's pairs, loaded even values first)."""
    x = _f64(x).copy()
    d = x.shape[-1]
    heads = x.shape[-2]
    rows = int(np.prod(x.shape[:-2], dtype=np.int64))
    w = _f64(w)
    assert w.shape == (d,)
    if half > 0:
        cos = _f64(cos)
        sin = _f64(sin)
        assert cos.shape == sin.shape and cos.shape[1] == half
        table_rows = cos.shape[0]
        pos = np.ascontiguousarray(np.broadcast_to(np.asarray(pos, dtype=np.int64),
                                                   x.shape[:-2])).reshape(-1)
    else:
        cos = sin = None
        table_rows = 0
        pos = None
    fn = _load().oracle_headprep_pairs if pairs else _load().oracle_headprep
    rc = fn(_ptr(x), rows, heads, d, _ptr(w), _ptr(cos), _ptr(sin), half, table_rows, _ptr(pos), float(eps))
    if rc != 0:
        raise ValueError("oracle_headprep rejected its arguments (code %d)" % rc)
    return x


def row_norm_rope(x, w, cos, sin, head: int, pos, eps: float) -> np.ndarray:
    """LTX's whole-row norm and rotary (gizml:netops, Functions > rowNormRopeInto) of
    x [rows, width], returned as a new f64 array; cos/sin [table_rows, width/2] or None
    (norm only); ``pos`` the table row of each row."""
    x = _f64(x).copy()
    rows, width = x.shape
    w = _f64(w)
    assert w.shape == (width,)
    if cos is not None:
        cos, sin = _f64(cos), _f64(sin)
        assert cos.shape == sin.shape and cos.shape[1] == width // 2
        table_rows = cos.shape[0]
        pos = np.ascontiguousarray(np.broadcast_to(np.asarray(pos, dtype=np.int64), (rows,)))
    else:
        cos = sin = pos = None
        table_rows = 0
    rc = _load().oracle_row_norm_rope(_ptr(x), rows, width, head, _ptr(w), _ptr(cos), _ptr(sin), table_rows,
                                      _ptr(pos), float(eps))
    if rc != 0:
        raise ValueError("oracle_row_norm_rope rejected its arguments (code %d)" % rc)
    return x


def _attention_shapes(q, k, v):
    batch, tq, hq, d = q.shape
    bk, tk, hkv, dk = k.shape
    bv, tv, hv, dv = v.shape
    assert bk == batch and bv == batch and tv == tk and hv == hkv and dk == d
    return batch, tq, tk, hq, hkv, d, dv


def attention(q, k, v, scale: float, causal: bool, lens=None) -> np.ndarray:
    """softmax(q k^T scale [+ causal mask]) v in f64 (gizml:netops, Functions > attention).
    q [B, tq, hq, d], k [B, tk, hkv, d], v [B, tk, hkv, dv] -> [B, tq, hq, dv]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    batch, tq, tk, hq, hkv, d, dv = _attention_shapes(q, k, v)
    out = np.zeros((batch, tq, hq, dv), dtype=np.float64)
    lens_a = None if lens is None else np.ascontiguousarray(np.asarray(lens, dtype=np.int64))
    rc = _load().oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), batch, tq, tk, hq,
                                  hkv, d, dv, float(scale), int(bool(causal)), _ptr(lens_a))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments (code %d)" % rc)
    return out


def attention_rows(q, k, v, scale: float, causal: bool, sel, lens=None) -> np.ndarray:
    """The attention output only for the query rows sel = [(b, i, h), ...] -> [nsel, dv]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    batch, tq, tk, hq, hkv, d, dv = _attention_shapes(q, k, v)
    sel = np.ascontiguousarray(np.asarray(sel, dtype=np.int64).reshape(-1, 3))
    out = np.zeros((sel.shape[0], dv), dtype=np.float64)
    lens_a = None if lens is None else np.ascontiguousarray(np.asarray(lens, dtype=np.int64))
    rc = _load().oracle_attention_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(out), batch, tq, tk,
                                       hq, hkv, d, dv, float(scale), int(bool(causal)),
                                       _ptr(lens_a), _ptr(sel), sel.shape[0])
    if rc != 0:
        raise ValueError("oracle_attention_rows rejected its arguments (code %d)" % rc)
    return out


def prefill(q, k, v, qw, kw, cos, sin, half: int, eps: float, pos0: int, scale: float,
            causal: bool = True, sel=None, prep: bool = True):
    """HeadPrep of q and k at positions pos0 + t (headPrepInPlace's row rule), then
    attention.  Returns (out, k_prepped); with ``sel`` only those query rows of out.
    With prep=False the inputs go to attention unchanged."""
    seq = q.shape[1]
    if prep:
        pos = (pos0 + np.arange(seq, dtype=np.int64))[None, :].repeat(q.shape[0], axis=0)
        qh = headprep(q, qw, cos, sin, half, pos, eps)
        kh = headprep(k, kw, cos, sin, half, pos, eps)
    else:
        qh, kh = _f64(q), _f64(k)
    if sel is None:
        out = attention(qh, kh, v, scale, causal)
    else:
        out = attention_rows(qh, kh, v, scale, causal, sel)
    return out, kh


def prefill_chunk(q, k_new, v_new, k_cache, v_cache, n_past: int, qw, kw, cos, sin, half: int,
                  eps: float, scale: float, causal: bool = True, sel=None, prep: bool = True,
                  prep_k: bool = True):
    """A chunk of tq new tokens against a cache holding n_past prepped rows: the chunk's
    keys are prepped at positions n_past + t and written with its values to cache rows
    n_past .. n_past + tq - 1, then the chunk's queries (prepped at positions n_past + i)
    attend the cache rows 0 .. n_past + tq - 1, causal aligned bottom-right (netops
    attention with tq < tk).  Returns (out, k_cache', v_cache') (copies, f64); with
    ``sel`` only those query rows of out.  prep=False: nothing is prepped;
    prep_k=False: k_new is taken as already prepped."""
    q, k_new, v_new = _f64(q), _f64(k_new), _f64(v_new)
    kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
    B, tq = q.shape[0], q.shape[1]
    pos = (n_past + np.arange(tq, dtype=np.int64))[None, :].repeat(B, axis=0)
    qh = headprep(q, qw, cos, sin, half, pos, eps) if prep else q
    kh = headprep(k_new, kw, cos, sin, half, pos, eps) if (prep and prep_k) else k_new
    kc[:, n_past:n_past + tq] = kh
    vc[:, n_past:n_past + tq] = v_new
    tk = n_past + tq
    if sel is None:
        out = attention(qh, kc[:, :tk], vc[:, :tk], scale, causal)
    else:
        out = attention_rows(qh, kc[:, :tk], vc[:, :tk], scale, causal, sel)
    return out, kc, vc


def prefill_chunk_ragged(q, k_new, v_new, k_cache, v_cache, past, qw, kw, cos, sin, half: int,
                         eps: float, scale: float, causal: bool = True, prep: bool = True,
                         prep_k: bool = True):
    """One engine step over sequences at different cache lengths (compute guide "Tensors,
    GPU kernels and AI models", Step 5: one step reads the prompt rows of many sequences):
    sequence b's chunk of tq tokens goes after its own past[b] cached rows, exactly as
    prefill_chunk with n_past = past[b] on that sequence alone.  Returns (out, k_cache',
    v_cache') (copies, f64)."""
    past = np.asarray(past, dtype=np.int64).reshape(-1)
    B = q.shape[0]
    assert past.shape[0] == B
    out = np.zeros(q.shape[:3] + (v_new.shape[3],), dtype=np.float64)
    kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
    for b in range(B):
        sl = slice(b, b + 1)
        ob, kb, vb = prefill_chunk(q[sl], k_new[sl], v_new[sl], kc[sl], vc[sl], int(past[b]), qw, kw, cos, sin,
                                   half, eps, scale, causal, prep=prep, prep_k=prep_k)
        out[b], kc[b], vc[b] = ob[0], kb[0], vb[0]
    return out, kc, vc


def attended_rows(qkv, heads: int, head: int, group: int = 0, queries: int = 0, prep=None):
    """attentionRows / attendedRows (gizml:netops, Functions > attentionRows): qkv [n, 3 heads
    head] holds each row's q, k and v; with ``prep`` (a dict qw, kw, cos, sin, half, eps and
    optionally pairs) q and k are prepped first, row r at table row r.  Query row i (the
    first ``queries`` rows, all when 0) attends the keys of its group of ``group`` rows (all
    rows when 0) with scale 1/sqrt(head) and no mask inside the group.  Returns (out [nq,
    heads head], q prepped [n, heads, head], k prepped [n, heads, head]) in f64."""
    x = _f64(qkv)
    n = x.shape[0]
    x = x.reshape(n, 3, heads, head)
    q, k, v = x[:, 0], x[:, 1], x[:, 2]
    if prep is not None:
        pos = np.arange(n, dtype=np.int64)
        args = (prep["cos"], prep["sin"], prep["half"], pos, prep["eps"])
        q = headprep(q, prep["qw"], *args, pairs=prep.get("pairs", False))
        k = headprep(k, prep["kw"], *args, pairs=prep.get("pairs", False))
    nq = queries if queries else n
    g = group if 0 < group < n else n
    out = np.zeros((nq, heads, head), dtype=np.float64)
    for lo in range(0, nq, g):
        hi = min(lo + g, n)
        qhi = min(lo + g, nq)
        out[lo:qhi] = attention(q[None, lo:qhi], k[None, lo:hi], v[None, lo:hi], 1.0 / np.sqrt(head), False)[0]
    return out.reshape(nq, heads * head), q, k


def kv_quantize(x, bits: int):
    """Quantised-cache coding of every head of x [..., d] (f32 values) in `bits` (8, 4, 2):
    returns (codes [..., d] int32, lo [...] f32, step [...] f32, k [...] int32 -- the chosen
    candidate), as oracle_kv_quantize defines it."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    d = x.shape[-1]
    units = int(np.prod(x.shape[:-1], dtype=np.int64))
    codes = np.zeros(x.shape, dtype=np.int32)
    lo = np.zeros(x.shape[:-1], dtype=np.float32)
    step = np.zeros(x.shape[:-1], dtype=np.float32)
    kk = np.zeros(x.shape[:-1], dtype=np.int32)
    fp = ctypes.POINTER(ctypes.c_float)
    ip = ctypes.POINTER(ctypes.c_int32)
    rc = _load().oracle_kv_quantize(x.ctypes.data_as(fp), units, d, int(bits), codes.ctypes.data_as(ip),
                                    lo.ctypes.data_as(fp), step.ctypes.data_as(fp), kk.ctypes.data_as(ip))
    if rc != 0:
        raise ValueError("oracle_kv_quantize rejected its arguments (code %d)" % rc)
    return codes, lo, step, kk


def kv_dequantize(codes, lo, step) -> np.ndarray:
    """The values a coded head gives back, lo + step * code, in f64."""
    return (np.asarray(lo, np.float64)[..., None] +
            np.asarray(step, np.float64)[..., None] * np.asarray(codes, np.float64))


def kv_pack(codes, bits: int) -> np.ndarray:
    """The stored bytes of codes [..., d]: each 32-bit little-endian word holds 32 / bits
    consecutive codes, code j of the word at bit (j mod 2) * 16 + (j // 2) * bits (even
    codes in the low half-word, odd ones in the high half-word).  -> uint8 [..., d bits / 8]."""
    codes = np.asarray(codes, dtype=np.uint64)
    per = 32 // bits
    d = codes.shape[-1]
    assert d % per == 0
    g = codes.reshape(codes.shape[:-1] + (d // per, per))
    j = np.arange(per, dtype=np.uint64)
    shift = (j % 2) * 16 + (j // 2) * bits
    words = (g << shift).sum(axis=-1).astype(np.uint32)
    return words.view(np.uint8).reshape(codes.shape[:-1] + (d * bits // 8,))


def kv_unpack(packed, bits: int, d: int) -> np.ndarray:
    """Inverse of kv_pack -> int32 codes [..., d]."""
    packed = np.ascontiguousarray(np.asarray(packed, dtype=np.uint8))
    per = 32 // bits
    words = packed.view(np.uint32).astype(np.uint64)
    j = np.arange(per, dtype=np.uint64)
    shift = (j % 2) * 16 + (j // 2) * bits
    g = (words[..., None] >> shift) & np.uint64((1 << bits) - 1)
    return g.reshape(packed.shape[:-1] + (d,)).astype(np.int32)


def decode(q, k_cache, v_cache, lens, pos, qw, cos, sin, half: int, eps: float,
           scale: float) -> np.ndarray:
    """One new query row per sequence: q [B, hq, d] prepped at table row pos[b], then
    attention over the first lens[b] rows of the (already prepped) cache
    [B, capacity, hkv, d].  Returns [B, hq, dv]."""
    q = _f64(q)
    qh = headprep(q[:, None], qw, cos, sin, half, np.asarray(pos, dtype=np.int64)[:, None], eps)
    out = attention(qh, k_cache, v_cache, scale, causal=False, lens=lens)
    return out[:, 0]


def paged_rows(pool, pages, length: int) -> np.ndarray:
    """The first `length` cache rows of one sequence out of a paged pool (compute guide
    "Tensors, GPU kernels and AI models", Step 5: the engine's KV pool): row j is row
    j mod page_rows of page pages[j // page_rows].  pool [num_pages, page_rows, ...]."""
    pool = np.asarray(pool)
    page_rows = pool.shape[1]
    j = np.arange(length)
    return pool[np.asarray(pages, dtype=np.int64)[j // page_rows], j % page_rows]


def gather_paged(pool, pages, lens) -> np.ndarray:
    """Every sequence's cache out of a paged pool: [B, max(lens), ...], rows past lens[b]
    zero (they are never attended)."""
    pool = np.asarray(pool)
    lens = [int(n) for n in lens]
    out = np.zeros((len(lens), max(1, max(lens))) + pool.shape[2:], dtype=pool.dtype)
    for b, n in enumerate(lens):
        out[b, :n] = paged_rows(pool, pages[b], n)
    return out


def decode_paged(q, k_pool, v_pool, pages, lens, pos, qw, cos, sin, half: int, eps: float,
                 scale: float) -> np.ndarray:
    """decode over the caches a paged pool [num_pages, page_rows, hkv, d] holds for each
    sequence (pages [B, max_pages])."""
    return decode(q, gather_paged(k_pool, pages, lens), gather_paged(v_pool, pages, lens), lens, pos, qw, cos, sin,
                  half, eps, scale)


def decode_q(q, k_codes, k_lo, k_step, v_codes, v_lo, v_step, lens, pos, qw, cos, sin, half: int,
             eps: float, scale: float) -> np.ndarray:
    """Decode against a quantised cache: the cache [B, capacity, hkv, d] gives back
    lo + step * code per head (kv_dequantize), then the decode above.  Codes unpacked."""
    return decode(q, kv_dequantize(k_codes, k_lo, k_step), kv_dequantize(v_codes, v_lo, v_step), lens, pos,
                  qw, cos, sin, half, eps, scale)


def int8_code(x):
    """Symmetric int8 coding of each unit x[..., :] (f32 values): (codes int8 [...], scale
    f32 [...[:-1]]) with scale amax / 127 and codes rint(x (1/scale)) clamped to +-127."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    n = x.shape[-1]
    units = int(np.prod(x.shape[:-1], dtype=np.int64))
    codes = np.zeros(x.shape, dtype=np.int8)
    scale = np.zeros(x.shape[:-1], dtype=np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    rc = _load().oracle_int8_code(x.ctypes.data_as(fp), units, n, codes.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)),
                                  scale.ctypes.data_as(fp))
    if rc != 0:
        raise ValueError("oracle_int8_code rejected its arguments (code %d)" % rc)
    return codes, scale


def e4m3_code(x):
    """E4M3 coding of each unit x[..., :] (f32 values): (values f32 [...] -- the E4M3 numbers,
    nearest with ties to even, of x (1/scale)), scale f32 [...[:-1]] = amax / 448)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    n = x.shape[-1]
    units = int(np.prod(x.shape[:-1], dtype=np.int64))
    vals = np.zeros(x.shape, dtype=np.float32)
    scale = np.zeros(x.shape[:-1], dtype=np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    rc = _load().oracle_e4m3_code(x.ctypes.data_as(fp), units, n, vals.ctypes.data_as(fp), scale.ctypes.data_as(fp))
    if rc != 0:
        raise ValueError("oracle_e4m3_code rejected its arguments (code %d)" % rc)
    return vals, scale


KEY_TILE = 64     # keys that share one int8 key scale (a tile of consecutive keys of a group)


def rows8_operands(qkv, heads: int, head: int, group: int = 0, queries: int = 0, prep=None):
    """The operands of attentionRows' quantized path (gizml:netops, Functions > attentionRows:
    Q K^T on INT8, P V on E4M3): HeadPrep of q and k (row r at table row r) in f64, rounded to
    f32; q coded in int8 per (row, head); k in int8 per (tile of 64 consecutive keys of a
    group, head); v in E4M3 per (group, head).  Returns a dict of the codes and, per row and
    head, the scales (q8, sq, k8, sk, v8 (E4M3 values as f32), sv) and the values they give
    back (q_back, k_back, v_back, f64 [rows, heads, head])."""
    x = np.asarray(qkv, dtype=np.float64)
    n = x.shape[0]
    x = x.reshape(n, 3, heads, head)
    q, k, v = x[:, 0], x[:, 1], x[:, 2]
    if prep is not None:
        pos = np.arange(n, dtype=np.int64)
        args = (prep["cos"], prep["sin"], prep["half"], pos, prep["eps"])
        q = headprep(q, prep["qw"], *args, pairs=prep.get("pairs", False))
        k = headprep(k, prep["kw"], *args, pairs=prep.get("pairs", False))
    nq = queries if queries else n
    g = group if 0 < group < n else n
    q32, k32, v32 = q[:nq].astype(np.float32), k.astype(np.float32), v.astype(np.float32)
    q8, sq = int8_code(q32)
    k8 = np.zeros((n, heads, head), np.int8)
    sk = np.zeros((n, heads), np.float32)
    v8 = np.zeros((n, heads, head), np.float32)
    sv = np.zeros((n, heads), np.float32)
    for lo in range(0, n, g):
        hi = min(lo + g, n)
        vals, s = e4m3_code(np.ascontiguousarray(v32[lo:hi].transpose(1, 0, 2)).reshape(heads, -1))
        v8[lo:hi] = vals.reshape(heads, hi - lo, head).transpose(1, 0, 2)
        sv[lo:hi] = s[None, :]
        for t0 in range(lo, hi, KEY_TILE):
            t1 = min(t0 + KEY_TILE, hi)
            c, s = int8_code(np.ascontiguousarray(k32[t0:t1].transpose(1, 0, 2)).reshape(heads, -1))
            k8[t0:t1] = c.reshape(heads, t1 - t0, head).transpose(1, 0, 2)
            sk[t0:t1] = s[None, :]
    return dict(q8=q8, sq=sq, k8=k8, sk=sk, v8=v8, sv=sv, q32=q32, k32=k32,
                q_back=q8.astype(np.float64) * sq[..., None], k_back=k8.astype(np.float64) * sk[..., None],
                v_back=v8.astype(np.float64) * sv[..., None])


def attended_rows8(ops, heads: int, head: int, group: int = 0, queries: int = 0):
    """attentionRows over the values 8-bit operands give back (rows8_operands), in f64 with
    an exact softmax: out [nq, heads head]; and the per-element sum_j p_j |v_j| (same
    shape), which bounds what rounding the weights p changes in out."""
    n = ops["k_back"].shape[0]
    nq = queries if queries else n
    g = group if 0 < group < n else n
    out = np.zeros((nq, heads, head))
    bound = np.zeros((nq, heads, head))
    qb, kb, vb = ops["q_back"], ops["k_back"], ops["v_back"]
    for lo in range(0, nq, g):
        hi, qhi = min(lo + g, n), min(lo + g, nq)
        args = (1.0 / np.sqrt(head), False)
        out[lo:qhi] = attention(qb[None, lo:qhi], kb[None, lo:hi], vb[None, lo:hi], *args)[0]
        bound[lo:qhi] = attention(qb[None, lo:qhi], kb[None, lo:hi], np.abs(vb[None, lo:hi]), *args)[0]
    return out.reshape(nq, heads * head), bound.reshape(nq, heads * head)
