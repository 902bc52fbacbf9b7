"""The C ABI on the CPU: the library loads, exports what include/attn.h declares, and
rejects bad arguments on the host before enqueuing anything (no GPU is touched: every
call below fails validation, so no pointer is ever dereferenced)."""
import ctypes
import os
import re

import pytest

import transformer_attention_headprep_amd as tah
from transformer_attention_headprep_amd import attn as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000       # a 16-byte aligned address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    return tah.load_library()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert declared == sorted(tah.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert lib.attn_status_str(code)
    assert lib.attn_supported(128, A.ATTN_BF16) == 1
    assert lib.attn_supported(64, A.ATTN_F32) == 1
    assert lib.attn_supported(96, A.ATTN_BF16) == 0
    assert lib.attn_supported(128, 7) == 0


def _prep(half=64, rows=4096, qw=FAKE, kw=FAKE, cos=FAKE, sin=FAKE, eps=1e-6, pairs=0, kmax=0.0):
    return A.attn_headprep_t(qw, kw, cos, sin, half, rows, eps, pairs, kmax)


def _prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE + (1 << 32), v=FAKE + (2 << 32), out=FAKE + (3 << 32), batch=2, seq=16,
             hq=8, hkv=2, d=128, qrs=1024, krs=256, vrs=256, ors=1024, pos0=0, prep=_prep(),
             causal=1, scale=0.088, dtype=A.ATTN_BF16)
    a.update(kw)
    prep = ctypes.byref(a["prep"]) if a["prep"] is not None else None
    return lib.attn_prefill(a["q"], a["k"], a["v"], a["out"], a["batch"], a["seq"], a["hq"], a["hkv"],
                            a["d"], a["qrs"], a["krs"], a["vrs"], a["ors"], a["pos0"], prep,
                            a["causal"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), A.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=5), A.ATTN_ERR_UNSUPPORTED),
    (dict(q=None), A.ATTN_ERR_ARG),
    (dict(v=None), A.ATTN_ERR_ARG),
    (dict(q=FAKE + 2), A.ATTN_ERR_ARG),                 # misaligned
    (dict(hq=6, hkv=4, qrs=768), A.ATTN_ERR_ARG),       # hq not a multiple of hkv
    (dict(hkv=0), A.ATTN_ERR_ARG),
    (dict(qrs=1000), A.ATTN_ERR_ARG),                   # stride smaller than the row
    (dict(krs=260), A.ATTN_ERR_ARG),                    # stride not a multiple of 8
    (dict(batch=-1), A.ATTN_ERR_ARG),
    (dict(prep=_prep(half=65)), A.ATTN_ERR_ARG),        # 2 * half > d
    (dict(prep=_prep(half=-1)), A.ATTN_ERR_ARG),
    (dict(prep=_prep(rows=15)), A.ATTN_ERR_ARG),        # positions past the table
    (dict(pos0=1, prep=_prep(rows=16)), A.ATTN_ERR_ARG),
    (dict(pos0=-1), A.ATTN_ERR_ARG),
    (dict(prep=_prep(cos=None)), A.ATTN_ERR_ARG),
    (dict(prep=_prep(qw=None)), A.ATTN_ERR_ARG),
    (dict(prep=_prep(eps=-1.0)), A.ATTN_ERR_ARG),
    (dict(prep=_prep(eps=float("nan"))), A.ATTN_ERR_ARG),
    (dict(prep=_prep(kmax=-1.0)), A.ATTN_ERR_ARG),
    (dict(prep=_prep(kmax=float("nan"))), A.ATTN_ERR_ARG),
    (dict(prep=_prep(kmax=float("inf"))), A.ATTN_ERR_ARG),
    (dict(scale=float("inf")), A.ATTN_ERR_ARG),
    (dict(scale=0.0), A.ATTN_ERR_ARG),
    (dict(scale=-0.1), A.ATTN_ERR_ARG),
    (dict(out=FAKE + 512), A.ATTN_ERR_ARG),             # out overlaps q
])
def test_prefill_rejects(lib, kw, code):
    assert _prefill(lib, **kw) == code
    assert lib.attn_last_error()


def test_key_bound(lib):
    """attn_key_bound (host only): sqrt(d) max|kw| (1 + 2^-7); -1 for bad arguments."""
    import numpy as np
    kw = np.array([0.5, -1.75, 1.25, 0.0] * 32, dtype=np.float32)
    got = lib.attn_key_bound(kw.ctypes.data, 128)
    assert got == pytest.approx(np.sqrt(128) * 1.75 * (1 + 2.0 ** -7), rel=1e-12)
    assert tah.key_bound(kw, 128) == got
    assert lib.attn_key_bound(None, 128) == -1.0
    assert lib.attn_key_bound(kw.ctypes.data, 0) == -1.0
    bad = kw.copy()
    bad[7] = np.inf
    assert np.isnan(lib.attn_key_bound(bad.ctypes.data, 128))


def test_key_bound_holds_for_headprep_rows():
    """Every key row the oracle's HeadPrep writes (then rounded to bf16) has norm within
    key_bound(kw); a row with all its mass on the largest weight comes within 1 % of it."""
    import numpy as np
    import oracle
    import synthetic
    rng = np.random.default_rng(17)
    d, half = 128, 64
    kw = rng.uniform(0.3, 1.7, d).astype(np.float32)
    kw[37] = -2.5
    x = rng.standard_normal((1, 300, 2, d)) * rng.uniform(0.01, 100, (1, 300, 2, 1))
    x[0, 0, 0] = 0.0
    x[0, 0, 0, 37] = 3.0                       # all mass on the largest |weight|
    x[0, 1, 1] = 1e-30                         # eps dominates: a tiny row
    cos, sin = synthetic.rope_tables(300, half, d, 1e4)
    k = synthetic.bf16_round(oracle.headprep(x, kw, cos, sin, half, np.arange(300)[None], 1e-6))
    norms = np.sqrt((k.astype(np.float64) ** 2).sum(-1))
    bound = tah.key_bound(kw, d)
    assert norms.max() <= bound
    assert norms[0, 0, 0] >= 0.99 * bound


def test_prefill_empty_is_a_no_op(lib):
    assert _prefill(lib, seq=0) == A.ATTN_OK
    assert _prefill(lib, batch=0) == A.ATTN_OK


def _prep_call(lib, **kw):
    a = dict(q=FAKE, k=FAKE + (1 << 32), batch=1, seq=8, hq=4, hkv=2, d=64, qrs=256, krs=128,
             pos0=0, prep=_prep(half=32), dtype=A.ATTN_F32)
    a.update(kw)
    prep = ctypes.byref(a["prep"]) if a["prep"] is not None else None
    return lib.attn_prep(a["q"], a["k"], a["batch"], a["seq"], a["hq"], a["hkv"], a["d"], a["qrs"],
                         a["krs"], a["pos0"], prep, a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None, k=None), A.ATTN_ERR_ARG),
    (dict(prep=None), A.ATTN_ERR_ARG),
    (dict(d=256, qrs=1024, krs=512), A.ATTN_ERR_UNSUPPORTED),
    (dict(prep=_prep(half=32, kw=None)), A.ATTN_ERR_ARG),
    (dict(pos0=4090, prep=_prep(half=32, rows=4096)), A.ATTN_ERR_ARG),
    (dict(k=FAKE + 64), A.ATTN_ERR_ARG),                 # k lands on q's heads
    (dict(prep=_prep(half=32, pairs=2)), A.ATTN_ERR_ARG),  # pairs is 0 or 1
    (dict(prep=_prep(half=33, pairs=1)), A.ATTN_ERR_ARG),  # 2 * half > d in either layout
])
def test_prep_rejects(lib, kw, code):
    assert _prep_call(lib, **kw) == code


def test_prep_empty_is_a_no_op(lib):
    assert _prep_call(lib, seq=0) == A.ATTN_OK


def _chunk(lib, **kw):
    a = dict(q=FAKE, kn=FAKE + (1 << 32), vn=FAKE + (2 << 32), kc=FAKE + (3 << 32), vc=FAKE + (4 << 32),
             out=FAKE + (5 << 32), batch=2, tq=16, hq=8, hkv=2, d=128, cap=1024, n_past=100,
             prep=_prep(rows=4096), causal=1, scale=0.088, dtype=A.ATTN_BF16, past=None)
    a.update(kw)
    prep = ctypes.byref(a["prep"]) if a["prep"] is not None else None
    return lib.attn_prefill_chunk(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["out"], a["batch"], a["tq"],
                                  a["hq"], a["hkv"], a["d"], a["cap"], a["n_past"], a["past"], prep, a["causal"],
                                  a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), A.ATTN_ERR_UNSUPPORTED),
    (dict(q=None), A.ATTN_ERR_ARG),
    (dict(kc=None), A.ATTN_ERR_ARG),
    (dict(vn=FAKE + (2 << 32) + 4), A.ATTN_ERR_ARG),      # misaligned
    (dict(hq=7), A.ATTN_ERR_ARG),                         # hq not a multiple of hkv
    (dict(n_past=-1), A.ATTN_ERR_ARG),
    (dict(n_past=1010), A.ATTN_ERR_ARG),                  # n_past + tq > capacity
    (dict(cap=0), A.ATTN_ERR_ARG),
    (dict(tq=-1), A.ATTN_ERR_ARG),
    (dict(prep=_prep(rows=115)), A.ATTN_ERR_ARG),         # table ends before n_past + tq
    (dict(prep=_prep(qw=None)), A.ATTN_ERR_ARG),
    (dict(scale=0.0), A.ATTN_ERR_ARG),
    (dict(out=FAKE + (3 << 32) + 4096), A.ATTN_ERR_ARG),  # out inside the k cache
    (dict(vc=FAKE + (3 << 32) + 8192), A.ATTN_ERR_ARG),   # the caches overlap
    (dict(kn=FAKE + (4 << 32) + 512), A.ATTN_ERR_ARG),    # new keys inside the v cache
    (dict(past=FAKE + (5 << 32) + 64), A.ATTN_ERR_ARG),   # per-sequence lengths inside out
    (dict(past=FAKE + (3 << 32) + 64), A.ATTN_ERR_ARG),   # per-sequence lengths inside a cache
    (dict(past=FAKE + (6 << 32), n_past=1010), A.ATTN_ERR_ARG),   # the bound + tq > capacity
])
def test_prefill_chunk_rejects(lib, kw, code):
    assert _chunk(lib, **kw) == code
    assert lib.attn_last_error()


def test_prefill_chunk_empty_is_a_no_op(lib):
    assert _chunk(lib, tq=0) == A.ATTN_OK
    assert _chunk(lib, batch=0) == A.ATTN_OK


def _decode(lib, **kw):
    # splits=4: the call needs a workspace, so every case below fails on the host.
    a = dict(q=FAKE, k=FAKE + (1 << 32), v=FAKE + (2 << 32), out=FAKE + (3 << 32), batch=32, hq=32,
             hkv=8, d=128, cap=4096, lens=FAKE + (4 << 32), pos=FAKE + (5 << 32), max_len=4096,
             max_pos=4096, prep=_prep(rows=4097), scale=0.088, splits=4, ws=FAKE + (6 << 32), ws_bytes=1 << 30,
             dtype=A.ATTN_BF16)
    a.update(kw)
    prep = ctypes.byref(a["prep"]) if a["prep"] is not None else None
    return lib.attn_decode(a["q"], a["k"], a["v"], a["out"], a["batch"], a["hq"], a["hkv"], a["d"],
                           a["cap"], a["lens"], a["pos"], a["max_len"], a["max_pos"], prep, a["scale"], a["splits"],
                           a["ws"], a["ws_bytes"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ws_bytes=1000), A.ATTN_ERR_WORKSPACE),
    (dict(ws=None), A.ATTN_ERR_WORKSPACE),
    (dict(lens=None), A.ATTN_ERR_ARG),
    (dict(pos=None), A.ATTN_ERR_ARG),
    (dict(max_len=4097), A.ATTN_ERR_ARG),
    (dict(max_len=0), A.ATTN_ERR_ARG),
    (dict(splits=5000), A.ATTN_ERR_ARG),
    (dict(splits=-2), A.ATTN_ERR_ARG),
    (dict(hq=30), A.ATTN_ERR_ARG),
    (dict(d=80), A.ATTN_ERR_UNSUPPORTED),
    (dict(cap=0, max_len=0), A.ATTN_ERR_ARG),
    (dict(out=FAKE + 64), A.ATTN_ERR_ARG),               # out overlaps q
    (dict(max_pos=4097), A.ATTN_ERR_ARG),                # the bound on pos lies past the table
    (dict(max_pos=-1), A.ATTN_ERR_ARG),
])
def test_decode_rejects(lib, kw, code):
    assert _decode(lib, **kw) == code


def test_decode_max_pos_is_checked_only_with_a_turn(lib):
    """Without a turning HeadPrep the positions are not read, so max_pos is not checked:
    the call goes on to fail on its missing workspace instead."""
    assert _decode(lib, ws=None, max_pos=99999, prep=_prep(half=0, cos=None, sin=None, rows=0)) == A.ATTN_ERR_WORKSPACE
    assert _decode(lib, ws=None, max_pos=99999, prep=None) == A.ATTN_ERR_WORKSPACE
    assert _decode(lib, ws=None, max_pos=99999) == A.ATTN_ERR_ARG


def _decode_paged(lib, **kw):
    # splits=4 and a bad argument in every case: each call fails on the host.
    a = dict(q=FAKE, k=FAKE + (1 << 32), v=FAKE + (2 << 32), out=FAKE + (3 << 32), batch=32, hq=32,
             hkv=8, d=128, num_pages=2048, page_rows=64, pages=FAKE + (7 << 32), max_pages=64,
             lens=FAKE + (4 << 32), pos=FAKE + (5 << 32), max_len=4096, max_pos=4096, prep=_prep(rows=4097),
             scale=0.088, splits=4, ws=FAKE + (6 << 32), ws_bytes=1 << 30, dtype=A.ATTN_BF16)
    a.update(kw)
    prep = ctypes.byref(a["prep"]) if a["prep"] is not None else None
    return lib.attn_decode_paged(a["q"], a["k"], a["v"], a["out"], a["batch"], a["hq"], a["hkv"], a["d"],
                                 a["num_pages"], a["page_rows"], a["pages"], a["max_pages"], a["lens"], a["pos"],
                                 a["max_len"], a["max_pos"], prep, a["scale"], a["splits"], a["ws"], a["ws_bytes"], a["dtype"],
                                 None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=A.ATTN_F32), A.ATTN_ERR_UNSUPPORTED),
    (dict(pages=None), A.ATTN_ERR_ARG),
    (dict(pages=FAKE + (7 << 32) + 2), A.ATTN_ERR_ARG),     # misaligned table
    (dict(page_rows=48), A.ATTN_ERR_ARG),                    # not a power of two
    (dict(page_rows=8, max_pages=512), A.ATTN_ERR_ARG),      # below 16
    (dict(num_pages=0), A.ATTN_ERR_ARG),
    (dict(num_pages=1 << 25), A.ATTN_ERR_ARG),               # num_pages * page_rows >= 2^31
    (dict(max_pages=63), A.ATTN_ERR_ARG),                    # max_len > max_pages * page_rows
    (dict(max_pages=0), A.ATTN_ERR_ARG),
    (dict(ws_bytes=1000), A.ATTN_ERR_WORKSPACE),
    (dict(lens=None), A.ATTN_ERR_ARG),
    (dict(out=FAKE + (7 << 32)), A.ATTN_ERR_ARG),            # out overlaps the page table
    (dict(max_pos=4097), A.ATTN_ERR_ARG),                    # past the table
])
def test_decode_paged_rejects(lib, kw, code):
    assert _decode_paged(lib, **kw) == code
    assert lib.attn_last_error()


def test_decode_q_paged_rejects(lib):
    def call(**kw):
        a = dict(bits=(4, 4), page_rows=64, pages=FAKE + (7 << 32), dtype=A.ATTN_BF16, ws_bytes=1000, max_pos=4096)
        a.update(kw)
        prep = _prep(rows=4097)
        return lib.attn_decode_q_paged(FAKE, FAKE + (1 << 32), FAKE + (2 << 32), FAKE + (3 << 32), FAKE + (4 << 32),
                                       FAKE + (5 << 32), 32, 32, 8, 128, 2048, a["page_rows"], a["bits"][0],
                                       a["bits"][1], a["pages"], 64, FAKE + (6 << 32), FAKE + (8 << 32), 4096,
                                       a["max_pos"], ctypes.byref(prep), 0.088, 4, FAKE + (9 << 32), a["ws_bytes"], a["dtype"], None)
    assert call() == A.ATTN_ERR_WORKSPACE
    assert call(bits=(8, 4)) == A.ATTN_ERR_ARG
    assert call(page_rows=100) == A.ATTN_ERR_ARG
    assert call(pages=None) == A.ATTN_ERR_ARG
    assert call(dtype=A.ATTN_F32) == A.ATTN_ERR_UNSUPPORTED
    assert call(max_pos=4097) == A.ATTN_ERR_ARG


def test_prefill_chunk_paged_rejects(lib):
    def call(**kw):
        a = dict(page_rows=64, pages=FAKE + (7 << 32), max_pages=64, n_past=3584, tq=512, dtype=A.ATTN_BF16,
                 scale=0.088)
        a.update(kw)
        prep = _prep(rows=4097)
        return lib.attn_prefill_chunk_paged(FAKE, FAKE + (1 << 32), FAKE + (2 << 32), FAKE + (3 << 32),
                                            FAKE + (4 << 32), FAKE + (5 << 32), 4, a["tq"], 32, 8, 128, 256,
                                            a["page_rows"], a["pages"], a["max_pages"], a["n_past"], None,
                                            ctypes.byref(prep), 1, a["scale"], a["dtype"], None)
    assert call(scale=0.0) == A.ATTN_ERR_ARG                  # every case fails on the host
    assert call(dtype=A.ATTN_F32) == A.ATTN_ERR_UNSUPPORTED
    assert call(page_rows=32, max_pages=128) == A.ATTN_ERR_ARG    # pages below 64 rows
    assert call(page_rows=96) == A.ATTN_ERR_ARG                   # not a power of two
    assert call(pages=None) == A.ATTN_ERR_ARG
    assert call(max_pages=63) == A.ATTN_ERR_ARG                   # n_past + tq > max_pages * page_rows
    assert call(n_past=-1) == A.ATTN_ERR_ARG
    assert lib.attn_last_error()


def test_decode_sizes(lib):
    # up to 8 kv heads with up to 8 q heads each: a block per (sequence, group of 512 / d
    # kv heads, key split) reads whole cache-row pieces; about one block per CU, at least
    # 256 keys per split
    assert lib.attn_decode_default_splits(32, 32, 8, 128, 4096) == 4      # 2 groups of 4 kv heads
    assert lib.attn_decode_default_splits(32, 32, 8, 64, 4096) == 8       # 1 group of 8
    assert lib.attn_decode_workspace_size(32, 32, 8, 128, 4096, 0) == 4 * 32 * 32 * 130 * 4
    assert lib.attn_decode_workspace_size(32, 32, 8, 128, 4096, 1) == 0
    assert lib.attn_decode_workspace_size(32, 32, 8, 128, 4096, 3) == 3 * 32 * 32 * 130 * 4
    assert lib.attn_decode_default_splits(1, 32, 8, 128, 4096) == 16
    assert lib.attn_decode_workspace_size(1, 32, 8, 128, 4096, 0) == 16 * 32 * 130 * 4
    assert lib.attn_decode_default_splits(1, 32, 8, 128, 100000) == 128
    assert lib.attn_decode_default_splits(256, 32, 8, 128, 4096) == 1
    # 16 q heads per kv head: blocks per (sequence, kv head, group of 8 q heads); 256 such
    # units already give every CU a block: one split, no workspace
    assert lib.attn_decode_default_splits(32, 64, 4, 128, 4096) == 1
    assert lib.attn_decode_workspace_size(32, 64, 4, 128, 4096, 0) == 0
    assert lib.attn_decode_workspace_size(0, 32, 8, 128, 4096, 0) == 0
    assert _decode(lib, batch=0) == A.ATTN_OK


def test_peak_library_exports_what_peak_h_declares():
    """libpeak.so (calibration kernels of the benchmark) loads without a GPU and exports
    every function include/peak.h declares; bad arguments are refused on the host."""
    src = open(os.path.join(ROOT, "include", "peak.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    declared = sorted(set(re.findall(r"\b(peak_[a-z0-9_]+)\s*\(", src)))
    assert declared == ["peak_mfma_bf16", "peak_mfma_bf16_flops", "peak_stream_read"]
    lib = ctypes.CDLL(os.path.join(ROOT, "transformer_attention_headprep_amd", "libpeak.so"))
    for name in declared:
        assert hasattr(lib, name), name
    lib.peak_mfma_bf16_flops.restype = ctypes.c_double
    lib.peak_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    assert lib.peak_mfma_bf16_flops(2, 3) == 2 * 4 * 3 * 8 * 2 * 32 * 32 * 16
    lib.peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.peak_mfma_bf16(0, 10, FAKE, None) == -1
    lib.peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.peak_stream_read(FAKE, 1000, FAKE, None) == -1       # not a multiple of 16
    assert lib.peak_stream_read(FAKE + 8, 1024, FAKE, None) == -1   # misaligned


def _row_norm(lib, **kw):
    a = dict(x=FAKE, rows=16, width=2048, head=64, rs=2048, w=FAKE + (1 << 32), cos=FAKE + (2 << 32),
             sin=FAKE + (3 << 32), eps=1e-6, dtype=A.ATTN_BF16)
    a.update(kw)
    return lib.attn_row_norm_rope(a["x"], a["rows"], a["width"], a["head"], a["rs"], a["w"], a["cos"],
                                  a["sin"], a["eps"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), A.ATTN_ERR_UNSUPPORTED),
    (dict(x=None), A.ATTN_ERR_ARG),
    (dict(w=None), A.ATTN_ERR_ARG),
    (dict(x=FAKE + 8), A.ATTN_ERR_ARG),                  # misaligned
    (dict(rows=-1), A.ATTN_ERR_ARG),
    (dict(width=2044, rs=2048), A.ATTN_ERR_ARG),         # width not a multiple of 8
    (dict(width=16384, rs=16384), A.ATTN_ERR_ARG),       # wider than 8192
    (dict(head=60), A.ATTN_ERR_ARG),                     # head not a multiple of 8
    (dict(head=96), A.ATTN_ERR_ARG),                     # head does not divide width
    (dict(rs=2040), A.ATTN_ERR_ARG),                     # stride below the width
    (dict(rs=2052), A.ATTN_ERR_ARG),                     # stride not a multiple of 8
    (dict(sin=None), A.ATTN_ERR_ARG),                    # cos without sin
    (dict(cos=FAKE + (2 << 32) + 4), A.ATTN_ERR_ARG),    # misaligned table
    (dict(eps=-1.0), A.ATTN_ERR_ARG),
    (dict(eps=float("inf")), A.ATTN_ERR_ARG),
    (dict(rows=1 << 24), A.ATTN_ERR_ARG),
])
def test_row_norm_rope_rejects(lib, kw, code):
    assert _row_norm(lib, **kw) == code
    assert lib.attn_last_error()


def test_row_norm_rope_empty_is_a_no_op(lib):
    assert _row_norm(lib, rows=0) == A.ATTN_OK
    assert _row_norm(lib, rows=0, cos=None, sin=None) == A.ATTN_OK


def _quant(lib, **kw):
    a = dict(x=FAKE, batch=2, seq=16, heads=8, d=128, rs=1024, bits=4, codes=FAKE + (1 << 32),
             params=FAKE + (2 << 32), capacity=64, row0=8, dtype=A.ATTN_BF16)
    a.update(kw)
    return lib.attn_kv_quantize(a["x"], a["batch"], a["seq"], a["heads"], a["d"], a["rs"], a["bits"], a["codes"],
                                a["params"], a["capacity"], a["row0"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96, rs=768), A.ATTN_ERR_UNSUPPORTED),
    (dict(bits=3), A.ATTN_ERR_ARG),
    (dict(bits=16), A.ATTN_ERR_ARG),
    (dict(x=None), A.ATTN_ERR_ARG),
    (dict(codes=None), A.ATTN_ERR_ARG),
    (dict(params=FAKE + (2 << 32) + 8), A.ATTN_ERR_ARG),   # misaligned
    (dict(row0=-1), A.ATTN_ERR_ARG),
    (dict(row0=49), A.ATTN_ERR_ARG),                        # row0 + seq > capacity
    (dict(capacity=0, row0=0), A.ATTN_ERR_ARG),
    (dict(rs=1000), A.ATTN_ERR_ARG),
    (dict(codes=FAKE + 4096), A.ATTN_ERR_ARG),              # codes overlap x
])
def test_kv_quantize_rejects(lib, kw, code):
    assert _quant(lib, **kw) == code
    assert lib.attn_last_error()


def test_kv_quantize_empty_is_a_no_op(lib):
    assert _quant(lib, seq=0) == A.ATTN_OK
    assert _quant(lib, batch=0) == A.ATTN_OK


def _decq(lib, **kw):
    a = dict(q=FAKE, kc=FAKE + (1 << 32), kp=FAKE + (2 << 32), vc=FAKE + (3 << 32), vp=FAKE + (4 << 32),
             out=FAKE + (5 << 32), batch=4, hq=32, hkv=8, d=128, cap=4096, kb=8, vb=8, lens=FAKE + (6 << 32),
             pos=FAKE + (7 << 32), max_len=4096, max_pos=4095, prep=_prep(), scale=0.088, splits=1, ws=None, wsb=0,
             dtype=A.ATTN_BF16)
    a.update(kw)
    prep = ctypes.byref(a["prep"]) if a["prep"] is not None else None
    return lib.attn_decode_q(a["q"], a["kc"], a["kp"], a["vc"], a["vp"], a["out"], a["batch"], a["hq"], a["hkv"],
                             a["d"], a["cap"], a["kb"], a["vb"], a["lens"], a["pos"], a["max_len"], a["max_pos"], prep,
                             a["scale"],
                             a["splits"], a["ws"], a["wsb"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=A.ATTN_F32), A.ATTN_ERR_UNSUPPORTED),       # bf16 q and out only
    (dict(d=96), A.ATTN_ERR_UNSUPPORTED),
    (dict(kb=8, vb=4), A.ATTN_ERR_ARG),                     # not an offered pair
    (dict(kb=2, vb=4), A.ATTN_ERR_ARG),
    (dict(kb=16, vb=16), A.ATTN_ERR_ARG),
    (dict(kc=None), A.ATTN_ERR_ARG),
    (dict(vp=FAKE + (4 << 32) + 4), A.ATTN_ERR_ARG),        # misaligned
    (dict(lens=None), A.ATTN_ERR_ARG),
    (dict(max_len=0), A.ATTN_ERR_ARG),
    (dict(max_len=4097), A.ATTN_ERR_ARG),
    (dict(hq=30), A.ATTN_ERR_ARG),
    (dict(scale=-1.0), A.ATTN_ERR_ARG),
    (dict(pos=None), A.ATTN_ERR_ARG),                       # turning HeadPrep needs pos
    (dict(splits=4), A.ATTN_ERR_WORKSPACE),                 # a workspace is needed and missing
    (dict(out=FAKE + 256), A.ATTN_ERR_ARG),                 # out overlaps q
    (dict(prep=_prep(pairs=3)), A.ATTN_ERR_ARG),
    (dict(max_pos=4096), A.ATTN_ERR_ARG),                   # the table has 4096 rows
])
def test_decode_q_rejects(lib, kw, code):
    assert _decq(lib, **kw) == code
    assert lib.attn_last_error()


def test_decode_q_default_splits(lib):
    # the decode workload's 256 (sequence, kv head) units: one round of 2 blocks per CU
    assert lib.attn_decode_q_default_splits(32, 32, 8, 4096, 8) == 2
    assert lib.attn_decode_q_default_splits(32, 32, 8, 4096, 4) == 3
    assert lib.attn_decode_q_default_splits(32, 32, 8, 4096, 2) == 3
    assert lib.attn_decode_q_default_splits(4, 32, 8, 4096, 4) == 16      # at most max_len / 256
    assert lib.attn_decode_q_default_splits(4, 32, 8, 300, 4) == 2      # at least 256 keys a split
    assert lib.attn_decode_q_default_splits(32, 32, 8, 4096, 3) == 0     # not a width
    assert lib.attn_decode_q_default_splits(0, 32, 8, 4096, 8) == 0


def test_decode_q_empty_is_a_no_op(lib):
    assert _decq(lib, batch=0) == A.ATTN_OK


def test_rows8_layout(lib):
    total, off = A.rows8_layout(300, 4, 128, group=128, queries=200)
    # 3 groups of 128 rows (the last 44), 2 key tiles and 1 query tile a group
    sizes = dict(q8=200 * 4 * 128, sq=200 * 4 * 4, k8=300 * 4 * 128, sk=3 * 2 * 4 * 4, v8t=3 * 2 * 4 * 128 * 64,
                 sv=3 * 4 * 4, vmax=3 * 2 * 4 * 4)
    at = 0
    for part in A.ROWS8_PARTS:
        assert off[part] == at and at % 256 == 0
        at += (sizes[part] + 255) // 256 * 256
    assert total == at
    assert lib.attn_rows8_layout(300, 4, 96, 0, 0, None) == 0          # head not 64 or 128
    assert lib.attn_rows8_layout(300, 4, 128, 0, 301, None) == 0       # queries > n


def _rows8(lib, **kw):
    a = dict(qkv=FAKE, n=300, heads=4, head=128, group=0, queries=0, out=FAKE + (1 << 32), prep=_prep(),
             ws=FAKE + (2 << 32), wsb=1 << 30)
    a.update(kw)
    prep = ctypes.byref(a["prep"]) if a["prep"] is not None else None
    return lib.attn_rows8(a["qkv"], a["n"], a["heads"], a["head"], a["group"], a["queries"], a["out"], prep, a["ws"],
                          a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(head=96), A.ATTN_ERR_UNSUPPORTED),
    (dict(prep=_prep(half=32)), A.ATTN_ERR_UNSUPPORTED),      # split halves other than head / 2
    (dict(qkv=None), A.ATTN_ERR_ARG),
    (dict(out=None), A.ATTN_ERR_ARG),
    (dict(ws=None), A.ATTN_ERR_WORKSPACE),
    (dict(wsb=1000), A.ATTN_ERR_WORKSPACE),
    (dict(ws=FAKE + (2 << 32) + 8), A.ATTN_ERR_ARG),         # misaligned
    (dict(queries=301), A.ATTN_ERR_ARG),
    (dict(group=-1), A.ATTN_ERR_ARG),
    (dict(ws=FAKE + 4096), A.ATTN_ERR_ARG),                  # workspace overlaps qkv
    (dict(prep=_prep(rows=100)), A.ATTN_ERR_ARG),             # table shorter than n
])
def test_rows8_rejects(lib, kw, code):
    assert _rows8(lib, **kw) == code
    assert lib.attn_last_error()


def test_rows8_empty_is_a_no_op(lib):
    assert _rows8(lib, n=0) == A.ATTN_OK


def test_guarded_kernels_do_not_spill():
    """The kernels that count their own loads into LDS in vmcnt (bf16 prefill, whole-row
    decode) are built without register spills: the build's resource report says so (the
    build itself fails otherwise)."""
    from transformer_attention_headprep_amd import build as B
    if not os.path.exists(B.RESOURCE_REPORT):
        pytest.skip("library not built in this tree")
    rows = [line.split() for line in open(B.RESOURCE_REPORT) if line.strip()]
    guarded = [r for r in rows if any(k in r[1] for k in B.NO_SPILL[r[0]])]
    assert guarded, "no guarded kernel in the report"
    for r in guarded:
        assert r[3] == "vgpr_spill=0", r


def test_resource_report_parser_reads_spills():
    from transformer_attention_headprep_amd import build as B
    text = ("x.hip:1:1: remark: Function Name: _Z3fooi [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     VGPRs Spill: 94 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     SGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]\n")
    assert B.parse_resource_usage(text) == [("_Z3fooi", 256, 94, 3)]
