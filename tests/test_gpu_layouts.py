"""GPU parity of the image/video-model layouts against the f64 oracle: HeadPrep with
adjacent pairs (FLUX.3's rotary) through every entry point, packed-row attention with
block-diagonal groups and a query prefix (attn_rows), and the whole-row norm with a
per-head rotary (attn_row_norm_rope).  Tolerances as in tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
import transformer_attention_headprep_amd as tah
from gpu_util import assert_close, dev, host, require_gpu

pytestmark = pytest.mark.gpu


def _prep_dev(inp, half, pairs):
    cos = dev(inp["cos"][:, :half], "f32").contiguous() if half else None
    sin = dev(inp["sin"][:, :half], "f32").contiguous() if half else None
    return tah.HeadPrep(dev(inp["qw"], "f32"), dev(inp["kw"], "f32"), cos, sin, inp["eps"], pairs=pairs)


def _hp(x, w, inp, half, pos, pairs=True):
    return oracle.headprep(x, w, inp["cos"][:, :half], inp["sin"][:, :half], half, pos, inp["eps"], pairs=pairs)


# ------------------------------------------------------------------- adjacent pairs

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,half", [(64, 32), (128, 64), (128, 24), (64, 13), (128, 0)])
def test_prep_pairs_parity(dtype, d, half):
    require_gpu()
    w = synthetic.Workload("pp", "prefill", dtype, 2, 6, 2, 37, d, half, 1e4, 19)
    inp = synthetic.make_prefill(w)
    inp["cos"], inp["sin"] = synthetic.rope_tables(40, half, d, 1e4)
    q, k = dev(inp["q"], dtype), dev(inp["k"], dtype)
    tah.attn_prep(q, k, _prep_dev(inp, half, True), pos0=3)
    pos = (3 + np.arange(37))[None, :].repeat(2, 0)
    assert_close(host(q), _hp(inp["q"], inp["qw"], inp, half, pos), dtype, "pairs q")
    assert_close(host(k), _hp(inp["k"], inp["kw"], inp, half, pos), dtype, "pairs k")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,half", [(128, 64), (64, 32), (128, 40)])
def test_prefill_pairs(dtype, d, half):
    """attn_prefill with adjacent pairs: q goes through the prep pass into out first."""
    require_gpu()
    w = synthetic.Workload("fp", "prefill", dtype, 2, 8, 2, 211, d, half, 1e4, 23)
    inp = synthetic.make_prefill(w)
    inp["cos"], inp["sin"] = synthetic.rope_tables(216, half, d, 1e4)     # positions 5 .. 215
    q, k, v = dev(inp["q"], dtype), dev(inp["k"], dtype), dev(inp["v"], dtype)
    out = tah.attn_prefill(q, k, v, prep=_prep_dev(inp, half, True), pos0=5, causal=True, scale=w.scale)
    pos = (5 + np.arange(211))[None, :].repeat(2, 0)
    qh, kh = _hp(inp["q"], inp["qw"], inp, half, pos), _hp(inp["k"], inp["kw"], inp, half, pos)
    assert_close(host(out), oracle.attention(qh, kh, inp["v"], w.scale, True), dtype, "prefill pairs")
    assert_close(host(k), kh, dtype, "k prepped in place")


def test_prefill_chunk_pairs():
    require_gpu()
    n_past, tq, half = 150, 90, 64
    w = synthetic.Workload("cp", "prefill", "bf16", 2, 8, 2, n_past + tq, 128, half, 1e4, 29)
    inp = synthetic.make_prefill(w)
    pos = np.arange(n_past + tq)[None].repeat(2, 0)
    kh = _hp(inp["k"], inp["kw"], inp, half, pos)
    qh = _hp(inp["q"], inp["qw"], inp, half, pos)
    kc = np.zeros((2, n_past + tq + 4, 2, 128))
    vc = np.zeros_like(kc)
    kc[:, :n_past] = synthetic.bf16_round(kh[:, :n_past])
    vc[:, :n_past] = inp["v"][:, :n_past]
    kcd, vcd = dev(kc, "bf16"), dev(vc, "bf16")
    sl = slice(n_past, None)
    out = tah.attn_prefill_chunk(dev(inp["q"][:, sl], "bf16"), dev(inp["k"][:, sl], "bf16"),
                                 dev(inp["v"][:, sl], "bf16"), kcd, vcd, n_past,
                                 prep=_prep_dev(inp, half, True), causal=True, scale=w.scale)
    kc_ref = kc[:, :n_past + tq].copy()
    kc_ref[:, n_past:] = kh[:, n_past:]
    ref = oracle.attention(qh[:, sl], kc_ref, inp["v"], w.scale, True)
    assert_close(host(out), ref, "bf16", "chunk pairs")
    assert_close(host(kcd)[:, n_past:n_past + tq], kh[:, n_past:], "bf16", "appended keys")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_pairs(dtype):
    require_gpu()
    B, cap, hq, hkv, d, half = 4, 700, 16, 4, 128, 64
    w = synthetic.Workload("dp", "decode", dtype, B, hq, hkv, cap, d, half, 1e4, 31)
    inp = synthetic.make_decode(w)
    lens = np.array([700, 1, 333, 512])
    pos = np.array([700, 5, 333, 1000])
    inp["cos"], inp["sin"] = synthetic.rope_tables(1024, half, d, 1e4)
    kpos = np.arange(cap)[None].repeat(B, 0)
    kc = synthetic.to_storage(_hp(inp["k_raw"], inp["kw"], inp, half, kpos), dtype)
    out = tah.attn_decode(dev(inp["q"], dtype), dev(kc, dtype), dev(inp["v"], dtype),
                          torch.tensor(lens, dtype=torch.int32, device="cuda:0"),
                          torch.tensor(pos, dtype=torch.int32, device="cuda:0"), cap,
                          prep=_prep_dev(inp, half, True), scale=w.scale)
    qh = _hp(inp["q"][:, None], inp["qw"], inp, half, pos[:, None])
    ref = oracle.attention(qh, kc, inp["v"], w.scale, False, lens=lens)[:, 0]
    assert_close(host(out), ref, dtype, "decode pairs")


# ---------------------------------------------------------------- packed rows (attn_rows)

def _rows_inputs(n, heads, head, half, dtype, seed):
    rng = np.random.default_rng(seed)
    qkv = synthetic.to_storage(rng.standard_normal((n, 3 * heads * head)), dtype)
    qw = rng.uniform(0.5, 1.5, head).astype(np.float32)
    kw = rng.uniform(0.5, 1.5, head).astype(np.float32)
    cos, sin = synthetic.rope_tables(n, half, head, 1e4)
    return qkv, dict(qw=qw, kw=kw, cos=cos, sin=sin, half=half, eps=1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n,heads,head,group,queries,prep,pairs", [
    (300, 4, 128, 0, 0, True, False),      # every row sees every row
    (300, 4, 64, 128, 0, True, True),      # groups of 128, the last one 44 rows
    (300, 2, 128, 100, 150, True, False),  # queries end inside the second group
    (257, 3, 64, 0, 200, False, False),    # a query prefix, no HeadPrep
    (130, 2, 128, 1, 0, True, False),      # groups of one row: each row sees itself
    (64, 1, 128, 64, 64, True, True),      # one whole group
])
def test_rows_parity(dtype, n, heads, head, group, queries, prep, pairs):
    require_gpu()
    qkv, p = _rows_inputs(n, heads, head, head // 2, dtype, seed=n + group + queries)
    p["pairs"] = pairs
    t = dev(qkv, dtype)
    hp = tah.HeadPrep(dev(p["qw"], "f32"), dev(p["kw"], "f32"), dev(p["cos"], "f32"), dev(p["sin"], "f32"),
                      p["eps"], pairs=pairs) if prep else None
    out = tah.attn_rows(t, heads, head, group=group, queries=queries, prep=hp)
    ref, qh, kh = oracle.attended_rows(qkv, heads, head, group, queries, p if prep else None)
    assert_close(host(out), ref, dtype, "attn_rows")
    nq = queries if queries else n
    got = host(t).reshape(n, 3, heads, head)
    src = qkv.reshape(n, 3, heads, head)
    assert_close(got[:nq, 0], qh[:nq], dtype, "q prepped in place")
    assert_close(got[:, 1], kh, dtype, "k prepped in place")
    np.testing.assert_array_equal(got[nq:, 0], src[nq:, 0])     # q rows that are not queries
    np.testing.assert_array_equal(got[:, 2], src[:, 2])         # v never written
    if group == 1:   # a query that sees only its own key returns its own value
        assert_close(host(out), src[:nq, 2].reshape(nq, -1), dtype, "group of one")


def test_rows_image_model_shape_sampled():
    """4096 image + 512 text rows of 24 heads of 128 with FLUX.3's pairs (the joint block's
    attention at 1024 x 1024): sampled query rows against the oracle."""
    require_gpu()
    n, heads, head = 4608, 24, 128
    qkv, p = _rows_inputs(n, heads, head, 64, "bf16", seed=37)
    p["pairs"] = True
    t = dev(qkv, "bf16")
    hp = tah.HeadPrep(dev(p["qw"], "f32"), dev(p["kw"], "f32"), dev(p["cos"], "f32"), dev(p["sin"], "f32"),
                      p["eps"], pairs=True)
    out = host(tah.attn_rows(t, heads, head, prep=hp)).reshape(n, heads, head)
    x = qkv.reshape(n, 3, heads, head)
    pos = np.arange(n)
    qh = oracle.headprep(x[:, 0], p["qw"], p["cos"], p["sin"], 64, pos, p["eps"], pairs=True)
    kh = oracle.headprep(x[:, 1], p["kw"], p["cos"], p["sin"], 64, pos, p["eps"], pairs=True)
    rng = np.random.default_rng(3)
    rows = sorted({0, 1, 127, 128, 4095, 4096, n - 1} | set(rng.integers(0, n, 20).tolist()))
    sel = np.array([(0, r, (r * 7 + j) % heads) for r in rows for j in (0, 11)], dtype=np.int64)
    ref = oracle.attention_rows(qh[None], kh[None], x[None, :, 2], 1 / np.sqrt(head), False, sel)
    assert_close(out[sel[:, 1], sel[:, 2]], ref, "bf16", "sampled rows")


# ------------------------------------------------------- whole-row norm (attn_row_norm_rope)

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,width,head,extra,table", [
    (37, 2048, 64, 0, True),      # LTX-Video's q width, 32 heads of 64
    (5, 4096, 128, 8, True),      # row stride past the width
    (3, 8192, 128, 0, True),      # the widest row
    (50, 520, 40, 0, True),       # 13 heads of 40, a width that is no power of two
    (17, 24, 8, 16, False),       # the norm only
    (9, 2048, 2048, 0, True),     # one head spanning the row
])
def test_row_norm_rope_parity(dtype, rows, width, head, extra, table):
    require_gpu()
    rng = np.random.default_rng(rows * 7 + width)
    buf = synthetic.to_storage(rng.standard_normal((rows, width + extra)), dtype)
    wt = rng.uniform(0.5, 1.5, width).astype(np.float32)
    ang = rng.uniform(-np.pi, np.pi, (rows, width // 2))
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    t = dev(buf, dtype)
    x = t[:, :width]
    tah.attn_row_norm_rope(x, dev(wt, "f32"), 1e-6, dev(cos, "f32") if table else None,
                           dev(sin, "f32") if table else None, head=head)
    ref = oracle.row_norm_rope(buf[:, :width], wt, cos if table else None, sin if table else None, head,
                               np.arange(rows), 1e-6)
    got = host(t)
    assert_close(got[:, :width], ref, dtype, "row norm")
    np.testing.assert_array_equal(got[:, width:], buf[:, width:])   # past the width: untouched
