"""Pins of the f64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a hand-worked
example, a library routine (torch's rms_norm and scaled_dot_product_attention, numpy's
complex product), a closed form, or an invariant of the definition.  Together they are
chosen so that a dropped term, a wrong sign, a wrong pairing or table row, a missing
scale, a misaligned mask or a wrong head grouping fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synthetic
from kv_util import np_quantize

RNG = np.random.default_rng(1234)


def _angles_tables(rows, half, d, base=1e4):
    """Exact f64 tables (no f32 rounding), for the relative-position invariant."""
    p = np.arange(rows, dtype=np.float64)[:, None]
    i = np.arange(half, dtype=np.float64)[None, :]
    ang = p * base ** (-2.0 * i / d)
    return np.cos(ang), np.sin(ang)


def _torch_rmsnorm(x, w, eps):
    xt = torch.from_numpy(np.asarray(x, dtype=np.float64))
    return F.rms_norm(xt, (xt.shape[-1],), weight=torch.from_numpy(np.asarray(w, np.float64)),
                      eps=eps).numpy()


# ---------------------------------------------------------------------------- HeadPrep

def test_headprep_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "headprep_worked.json")) as f:
        spec = json.load(f)
    for case in spec["cases"]:
        x = np.array(case["x"])[None, None, :]
        half = case["half"]
        cos = np.array(case["cos"], dtype=np.float64).reshape(-1, half) if half else None
        sin = np.array(case["sin"], dtype=np.float64).reshape(-1, half) if half else None
        got = oracle.headprep(x, case["w"], cos, sin, half, [case["pos"]], case["eps"])
        np.testing.assert_allclose(got[0, 0], case["expect"], rtol=0, atol=1e-15,
                                   err_msg=case["name"])


@pytest.mark.parametrize("d", [4, 64, 128])
def test_unit_rms_before_weight(d):
    """With w = 1 and no turn, each head's RMS is sqrt(ms / (ms + eps))."""
    eps = 1e-3
    x = RNG.standard_normal((7, 3, d)) * RNG.uniform(0.01, 10, (7, 3, 1))
    got = oracle.headprep(x, np.ones(d), None, None, 0, 0, eps)
    ms = (x ** 2).mean(-1)
    np.testing.assert_allclose(np.sqrt((got ** 2).mean(-1)), np.sqrt(ms / (ms + eps)),
                               rtol=1e-13, atol=0)


def test_norm_weight_matches_torch_rms_norm():
    """half = 0 reduces HeadPrep to torch's rms_norm with the same weight and eps."""
    d = 64
    x = RNG.standard_normal((5, 4, d)) * 3
    w = RNG.uniform(0.5, 1.5, d)
    for eps in (0.0, 1e-6, 0.25):
        got = oracle.headprep(x, w, None, None, 0, 0, eps)
        np.testing.assert_allclose(got, _torch_rmsnorm(x, w, eps), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("d,half", [(64, 32), (128, 64), (128, 32), (10, 3)])
def test_turn_is_complex_multiplication(d, half):
    """The split-half turn of pair (e, e+half) is (a + ib) * (cos + i sin)."""
    rows, heads = 6, 3
    x = RNG.standard_normal((rows, heads, d))
    w = RNG.uniform(0.5, 1.5, d)
    ang = RNG.uniform(-math.pi, math.pi, (9, half))
    cos, sin = np.cos(ang), np.sin(ang)
    pos = RNG.integers(0, 9, rows)
    got = oracle.headprep(x, w, cos, sin, half, pos, 1e-6)
    n = _torch_rmsnorm(x, w, 1e-6)
    z = (n[..., :half] + 1j * n[..., half:2 * half]) * np.exp(1j * ang[pos])[:, None, :]
    np.testing.assert_allclose(got[..., :half], z.real, atol=1e-14)
    np.testing.assert_allclose(got[..., half:2 * half], z.imag, atol=1e-14)
    np.testing.assert_allclose(got[..., 2 * half:], n[..., 2 * half:], rtol=0, atol=1e-14)


def test_pair_norm_preserved_and_position_zero_identity():
    d, half = 128, 64
    x = RNG.standard_normal((4, 2, d))
    w = RNG.uniform(0.5, 1.5, d)
    cos, sin = synthetic.rope_tables(64, half, d, 1e4)
    pos = np.array([0, 5, 17, 63])
    got = oracle.headprep(x, w, cos.astype(np.float64), sin.astype(np.float64), half, pos, 1e-6)
    plain = oracle.headprep(x, w, None, None, 0, 0, 1e-6)
    # |cos|^2 + |sin|^2 of the f32 table entries is 1 within f32 rounding
    c2s2 = cos.astype(np.float64) ** 2 + sin.astype(np.float64) ** 2
    before = plain[..., :half] ** 2 + plain[..., half:] ** 2
    after = got[..., :half] ** 2 + got[..., half:] ** 2
    np.testing.assert_allclose(after, before * c2s2[pos][:, None, :], rtol=1e-13)
    np.testing.assert_allclose(np.abs(c2s2 - 1).max(), 0, atol=3e-7)
    # position 0: cos = 1, sin = 0 exactly, so the turn is the identity
    np.testing.assert_array_equal(got[0], plain[0])


def test_scale_invariance():
    """prep(c x) = prep(x) up to eps: why scaled outlier keys are inert after HeadPrep."""
    d, half = 128, 64
    x = RNG.standard_normal((3, 2, d))
    w = RNG.uniform(0.5, 1.5, d)
    cos, sin = _angles_tables(8, half, d)
    a = oracle.headprep(x, w, cos, sin, half, [1, 4, 7], 1e-6)
    b = oracle.headprep(8.0 * x, w, cos, sin, half, [1, 4, 7], 1e-6)
    assert np.abs(a - b).max() < 1e-5
    assert np.abs(a - b).max() > 0  # eps really is in the formula


def test_relative_position():
    """A q.k score depends on the two positions only through their difference."""
    d, half = 64, 32
    cos, sin = _angles_tables(300, half, d)
    q = RNG.standard_normal((1, 1, d))
    k = RNG.standard_normal((1, 1, d))
    w = RNG.uniform(0.5, 1.5, d)
    scores = []
    for s in (0, 13, 100, 250):
        qh = oracle.headprep(q, w, cos, sin, half, [s + 40], 1e-6)
        kh = oracle.headprep(k, w, cos, sin, half, [s + 7], 1e-6)
        scores.append(float((qh * kh).sum()))
    np.testing.assert_allclose(scores, scores[0], rtol=0, atol=1e-11)


def test_headprep_rejects_bad_arguments():
    x = np.zeros((2, 1, 8))
    cos = np.ones((3, 4))
    with pytest.raises(ValueError):
        oracle.headprep(x, np.ones(8), cos, cos, 4, [0, 3], 1e-6)   # position past the table
    with pytest.raises(ValueError):
        oracle.headprep(x, np.ones(8), np.ones((3, 5)), np.ones((3, 5)), 5, [0, 1], 1e-6)


# --------------------------------------------------------------------------- attention

def test_attention_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "attention_worked.json")) as f:
        spec = json.load(f)
    k = np.array(spec["k"])[None]      # [1, tk, hkv, d]
    v = np.array(spec["v"])[None]
    for case in spec["cases"]:
        q = np.tile(np.array(spec["q_row"]), (1, case["tq"], spec["hq"], 1))
        got = oracle.attention(q, k, v, spec["scale"], case["causal"])
        np.testing.assert_allclose(got[0], np.array(case["expect"], dtype=np.float64),
                                   rtol=0, atol=1e-14, err_msg=case["name"])


def _bottom_right_mask(tq, tk):
    i = np.arange(tq)[:, None]
    j = np.arange(tk)[None, :]
    return j <= i + tk - tq


@pytest.mark.parametrize("tq,tk,causal", [(6, 6, True), (6, 6, False), (3, 9, True),
                                          (1, 9, True), (5, 8, False)])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (6, 1)])
def test_attention_matches_torch_sdpa(tq, tk, causal, hq, hkv):
    """torch's SDPA in f64 with an explicit bottom-right mask and grouped heads."""
    b, d, dv = 2, 8, 5
    q = RNG.standard_normal((b, tq, hq, d))
    k = RNG.standard_normal((b, tk, hkv, d))
    v = RNG.standard_normal((b, tk, hkv, dv))
    scale = 0.37
    got = oracle.attention(q, k, v, scale, causal)
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, dim=1)
    mask = torch.from_numpy(_bottom_right_mask(tq, tk)) if causal else None
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    np.testing.assert_allclose(got, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-13)


def test_softmax_weights_sum_to_one():
    q = RNG.standard_normal((2, 9, 2, 16)) * 3
    k = RNG.standard_normal((2, 9, 1, 16)) * 3
    v = np.ones((2, 9, 1, 4))
    got = oracle.attention(q, k, v, 0.5, True)
    np.testing.assert_allclose(got, 1.0, rtol=0, atol=1e-14)


def test_one_key_returns_v():
    q = RNG.standard_normal((3, 1, 2, 16))
    k = RNG.standard_normal((3, 1, 1, 16))
    v = RNG.standard_normal((3, 1, 1, 7))
    got = oracle.attention(q, k, v, 0.125, True)
    np.testing.assert_array_equal(got, np.repeat(v, 2, axis=2))


def test_zero_query_gives_prefix_means():
    """q = 0: all scores 0, so causal row i is the mean of v rows 0..i (closed form)."""
    s, d = 11, 8
    q = np.zeros((1, s, 1, d))
    k = RNG.standard_normal((1, s, 1, d))
    v = RNG.standard_normal((1, s, 1, 3))
    got = oracle.attention(q, k, v, 1.0, True)
    means = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, s + 1)[:, None]
    np.testing.assert_allclose(got[0, :, 0], means, atol=1e-15)


def test_causality():
    """Changing keys or values after row i leaves rows up to i exactly unchanged."""
    s, d = 12, 16
    q = RNG.standard_normal((1, s, 2, d))
    k = RNG.standard_normal((1, s, 2, d))
    v = RNG.standard_normal((1, s, 2, d))
    a = oracle.attention(q, k, v, 0.25, True)
    k2, v2 = k.copy(), v.copy()
    k2[:, 7:] = RNG.standard_normal(k2[:, 7:].shape)
    v2[:, 7:] = RNG.standard_normal(v2[:, 7:].shape)
    b = oracle.attention(q, k2, v2, 0.25, True)
    np.testing.assert_array_equal(a[:, :7], b[:, :7])
    assert np.abs(a[:, 7:] - b[:, 7:]).max() > 1e-3


def test_grouped_heads_equal_repeated_heads():
    q = RNG.standard_normal((2, 10, 8, 16))
    k = RNG.standard_normal((2, 10, 2, 16))
    v = RNG.standard_normal((2, 10, 2, 16))
    a = oracle.attention(q, k, v, 0.25, True)
    b = oracle.attention(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), 0.25, True)
    np.testing.assert_array_equal(a, b)


def test_dominant_key():
    q = np.zeros((1, 1, 1, 4))
    q[..., 0] = 1.0
    k = RNG.standard_normal((1, 6, 1, 4)) * 0.1
    k[0, 3, 0, 0] = 100.0
    v = RNG.standard_normal((1, 6, 1, 4))
    got = oracle.attention(q, k, v, 1.0, False)
    np.testing.assert_allclose(got[0, 0, 0], v[0, 3, 0], atol=1e-30 + 1e-40)


def test_lens_equal_truncated_cache_and_empty_rows_are_zero():
    q = RNG.standard_normal((3, 1, 4, 16))
    k = RNG.standard_normal((3, 20, 2, 16))
    v = RNG.standard_normal((3, 20, 2, 16))
    lens = [20, 7, 0]
    got = oracle.attention(q, k, v, 0.25, False, lens=lens)
    for b, n in enumerate(lens[:2]):
        ref = oracle.attention(q[b:b + 1], k[b:b + 1, :n], v[b:b + 1, :n], 0.25, False)
        np.testing.assert_array_equal(got[b], ref[0])
    np.testing.assert_array_equal(got[2], 0.0)


def test_rows_sample_equals_full():
    q = RNG.standard_normal((2, 33, 4, 16))
    k = RNG.standard_normal((2, 33, 2, 16))
    v = RNG.standard_normal((2, 33, 2, 16))
    full = oracle.attention(q, k, v, 0.25, True)
    sel = [(0, 0, 0), (1, 32, 3), (0, 17, 2), (1, 5, 1)]
    got = oracle.attention_rows(q, k, v, 0.25, True, sel)
    for r, (b, i, h) in enumerate(sel):
        np.testing.assert_array_equal(got[r], full[b, i, h])


# ----------------------------------------------------- HeadPrep variants (adjacent pairs)

def _even_first(x, half):
    """Permutation reading the first 2*half values of a head even ones first."""
    idx = np.concatenate([np.arange(0, 2 * half, 2), np.arange(1, 2 * half, 2), np.arange(2 * half, x.shape[-1])])
    return idx


@pytest.mark.parametrize("d,half", [(16, 8), (16, 5), (8, 0), (64, 32), (64, 24)])
def test_pairs_are_split_halves_of_the_even_first_reading(d, half):
    """FLUX.3's pairs "loaded even values first": HeadPrep with adjacent pairs is the
    split-halves HeadPrep of the values read even ones first (weights read the same
    way), put back in place."""
    x = RNG.standard_normal((5, 3, d))
    w = RNG.uniform(0.5, 1.5, d)
    cos, sin = _rand_tables(9, half)
    pos = np.array([0, 8, 3, 5, 1])
    idx = _even_first(x, half)
    got = oracle.headprep(x, w, cos, sin, half, pos, 1e-6, pairs=True)
    ref = np.empty_like(got)
    ref[..., idx] = oracle.headprep(x[..., idx], w[idx], cos, sin, half, pos, 1e-6)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)


def test_pairs_turn_is_complex_multiplication():
    """Pair (2i, 2i+1) as the complex number x_2i + i x_2i+1 times e^{i theta_i}."""
    d, half = 12, 6
    x = RNG.standard_normal((4, 2, d))
    ang = RNG.uniform(-np.pi, np.pi, (4, half))
    got = oracle.headprep(x, np.ones(d), np.cos(ang), np.sin(ang), half, np.arange(4), 0.0, pairs=True)
    n = x / np.sqrt((x ** 2).mean(-1, keepdims=True))
    z = (n[..., 0::2] + 1j * n[..., 1::2]) * np.exp(1j * ang)[:, None, :]
    np.testing.assert_allclose(got[..., 0::2], z.real, rtol=0, atol=1e-13)
    np.testing.assert_allclose(got[..., 1::2], z.imag, rtol=0, atol=1e-13)


# --------------------------------------------------- whole-row norm and rotary (LTX)

def _rand_tables(rows, half):
    ang = RNG.uniform(-np.pi, np.pi, (rows, half))
    return np.cos(ang), np.sin(ang)


def test_row_norm_rope_of_one_head_is_headprep():
    """With width = head the whole-row norm is the head's norm: rowNormRopeInto equals
    HeadPrep (split halves, half = head / 2) with w as the norm weight."""
    rows, head = 6, 16
    x = RNG.standard_normal((rows, head))
    w = RNG.uniform(0.5, 1.5, head)
    cos, sin = _rand_tables(10, head // 2)
    pos = np.array([3, 0, 9, 1, 4, 4])
    got = oracle.row_norm_rope(x, w, cos, sin, head, pos, 1e-6)
    ref = oracle.headprep(x[:, None, :], w, cos, sin, head // 2, pos, 1e-6)[:, 0, :]
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)


def test_row_norm_rope_equal_heads_is_headprep_per_head():
    """Rows whose heads all have the same sum of squares: the whole-row RMS equals each
    head's RMS, so every head comes out as HeadPrep with the row's table entries
    h*head/2 .. of that head (every head turns by its own angles)."""
    rows, heads, head = 4, 3, 8
    x = RNG.standard_normal((rows, heads, head))
    x /= np.sqrt((x ** 2).sum(-1, keepdims=True))          # every head: sum of squares 1
    w = RNG.uniform(0.5, 1.5, heads * head)
    cos, sin = _rand_tables(5, heads * head // 2)
    pos = np.array([4, 2, 0, 1])
    got = oracle.row_norm_rope(x.reshape(rows, -1), w, cos, sin, head, pos, 1e-6).reshape(rows, heads, head)
    for h in range(heads):
        tc, ts = cos[:, h * head // 2:(h + 1) * head // 2], sin[:, h * head // 2:(h + 1) * head // 2]
        ref = oracle.headprep(x[:, h:h + 1, :], w[h * head:(h + 1) * head], tc, ts, head // 2, pos, 1e-6)
        np.testing.assert_allclose(got[:, h], ref[:, 0], rtol=0, atol=1e-14)


def test_row_norm_unit_rms_and_pair_norms():
    """Without weight and tables the row comes out with RMS sqrt(ms / (ms + eps)); the
    turn keeps every (j, j + head/2) pair's norm."""
    rows, width, head, eps = 5, 48, 16, 1e-3
    x = RNG.standard_normal((rows, width))
    ms = (x ** 2).mean(-1)
    n = oracle.row_norm_rope(x, np.ones(width), None, None, head, None, eps)
    np.testing.assert_allclose(np.sqrt((n ** 2).mean(-1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)
    cos, sin = _rand_tables(rows, width // 2)
    t = oracle.row_norm_rope(x, np.ones(width), cos, sin, head, np.arange(rows), eps)
    a, b = n.reshape(rows, -1, 2, head // 2), t.reshape(rows, -1, 2, head // 2)
    np.testing.assert_allclose((b ** 2).sum(2), (a ** 2).sum(2), rtol=1e-12)


# -------------------------------------------------------------------------- the path

def test_decode_equals_prefill_row():
    """KV-cache equivalence: decode of position p over the cache prefill prepped
    (first p+1 rows) equals prefill's output row p."""
    w = synthetic.WORKLOADS["prefill_f32"]
    inp = synthetic.make_prefill(w, seq=24, batch=2)
    out, kh = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["qw"], inp["kw"], inp["cos"],
                             inp["sin"], w.half, w.eps, 0, w.scale, True)
    for p in (0, 9, 23):
        lens = np.full(2, p + 1)
        dec = oracle.decode(inp["q"][:, p], kh, inp["v"], lens, np.full(2, p), inp["qw"],
                            inp["cos"], inp["sin"], w.half, w.eps, w.scale)
        np.testing.assert_allclose(dec, out[:, p], rtol=0, atol=1e-14)


def test_chunked_prefill_equals_one_shot_prefill():
    """Chunked prefill (netops attention with tq < tk, bottom-right causal): feeding a
    sequence through the cache in chunks of 16, 1 and 23 tokens gives the one-shot
    prefill's output rows and leaves the one-shot prepped keys and the values in the
    cache; rows past the chunks stay as they were."""
    w = synthetic.WORKLOADS["prefill_f32"]
    inp = synthetic.make_prefill(w, seq=40, batch=2)
    full, kh = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["qw"], inp["kw"], inp["cos"],
                              inp["sin"], w.half, w.eps, 0, w.scale, True)
    cap = 48
    kc = np.full((2, cap, w.hkv, w.d), 7.0)
    vc = np.full((2, cap, w.hkv, w.d), -3.0)
    n_past = 0
    for tq in (16, 1, 23):
        sl = slice(n_past, n_past + tq)
        out, kc, vc = oracle.prefill_chunk(inp["q"][:, sl], inp["k"][:, sl], inp["v"][:, sl], kc, vc,
                                           n_past, inp["qw"], inp["kw"], inp["cos"], inp["sin"],
                                           w.half, w.eps, w.scale, True)
        np.testing.assert_allclose(out, full[:, sl], rtol=0, atol=1e-14)
        n_past += tq
    np.testing.assert_allclose(kc[:, :40], kh, rtol=0, atol=0)
    np.testing.assert_array_equal(vc[:, :40], inp["v"])
    assert (kc[:, 40:] == 7.0).all() and (vc[:, 40:] == -3.0).all()


def test_chunk_of_one_token_is_decode():
    """A chunk of one token at n_past is the decode of position n_past over the first
    n_past + 1 cache rows; a non-causal chunk sees every row up to n_past + tq - 1."""
    w = synthetic.WORKLOADS["prefill_f32"]
    inp = synthetic.make_prefill(w, seq=30, batch=2)
    _, kh = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["qw"], inp["kw"], inp["cos"],
                           inp["sin"], w.half, w.eps, 0, w.scale, True)
    n_past = 29
    out, kc, vc = oracle.prefill_chunk(inp["q"][:, 29:], inp["k"][:, 29:], inp["v"][:, 29:], kh, inp["v"],
                                       n_past, inp["qw"], inp["kw"], inp["cos"], inp["sin"], w.half,
                                       w.eps, w.scale, True)
    dec = oracle.decode(inp["q"][:, 29], kc, vc, np.full(2, 30), np.full(2, 29), inp["qw"], inp["cos"],
                        inp["sin"], w.half, w.eps, w.scale)
    np.testing.assert_allclose(out[:, 0], dec, rtol=0, atol=1e-14)
    # non-causal chunk of 4 at n_past 26: every query sees all 30 rows
    out_nc, kc2, vc2 = oracle.prefill_chunk(inp["q"][:, 26:], inp["k"][:, 26:], inp["v"][:, 26:], kh, inp["v"],
                                            26, inp["qw"], inp["kw"], inp["cos"], inp["sin"], w.half,
                                            w.eps, w.scale, False)
    for i in range(4):
        dec = oracle.decode(inp["q"][:, 26 + i], kc2, vc2, np.full(2, 30), np.full(2, 26 + i), inp["qw"],
                            inp["cos"], inp["sin"], w.half, w.eps, w.scale)
        np.testing.assert_allclose(out_nc[:, i], dec, rtol=0, atol=1e-14)


def test_ragged_chunks_equal_one_shot_prefill_per_sequence():
    """Sequences at different cache lengths in one step (compute guide, Step 5): sequence
    b's chunk after past[b] cached rows gives rows past[b] .. past[b] + tq - 1 of that
    sequence's one-shot causal prefill, writes its prepped keys and values at those rows,
    and leaves every later row as it was.  A non-causal chunk's query sees exactly the
    sequence's first past[b] + tq rows."""
    w = synthetic.WORKLOADS["prefill_f32"]
    past = np.array([0, 17, 29, 5], dtype=np.int64)
    tq, cap, B = 8, 48, 4
    inp = synthetic.make_prefill(w, seq=40, batch=B)
    kc = np.full((B, cap, w.hkv, w.d), 7.0)
    vc = np.full((B, cap, w.hkv, w.d), -3.0)
    fulls = []
    for b in range(B):
        T = int(past[b]) + tq
        full, kh = oracle.prefill(inp["q"][b:b + 1, :T], inp["k"][b:b + 1, :T], inp["v"][b:b + 1, :T], inp["qw"],
                                  inp["kw"], inp["cos"], inp["sin"], w.half, w.eps, 0, w.scale, True)
        fulls.append((full[0], kh[0]))
        kc[b, :past[b]] = kh[0, :past[b]]
        vc[b, :past[b]] = inp["v"][b, :past[b]]
    qn = np.stack([inp["q"][b, past[b]:past[b] + tq] for b in range(B)])
    kn = np.stack([inp["k"][b, past[b]:past[b] + tq] for b in range(B)])
    vn = np.stack([inp["v"][b, past[b]:past[b] + tq] for b in range(B)])
    out, kc2, vc2 = oracle.prefill_chunk_ragged(qn, kn, vn, kc, vc, past, inp["qw"], inp["kw"], inp["cos"],
                                                inp["sin"], w.half, w.eps, w.scale, True)
    for b in range(B):
        T = int(past[b]) + tq
        full, kh = fulls[b]
        np.testing.assert_allclose(out[b], full[past[b]:T], rtol=0, atol=1e-14)
        np.testing.assert_allclose(kc2[b, :T], kh, rtol=0, atol=0)
        np.testing.assert_array_equal(vc2[b, :T], inp["v"][b, :T])
        assert (kc2[b, T:] == 7.0).all() and (vc2[b, T:] == -3.0).all()
    # non-causal: query i of sequence b is the decode of position past[b] + i over T rows
    out_nc, kc3, vc3 = oracle.prefill_chunk_ragged(qn, kn, vn, kc, vc, past, inp["qw"], inp["kw"], inp["cos"],
                                                   inp["sin"], w.half, w.eps, w.scale, False)
    for b in range(B):
        T = int(past[b]) + tq
        for i in (0, tq - 1):
            dec = oracle.decode(qn[b:b + 1, i], kc3[b:b + 1], vc3[b:b + 1], np.array([T]),
                                np.array([past[b] + i]), inp["qw"], inp["cos"], inp["sin"], w.half, w.eps, w.scale)
            np.testing.assert_allclose(out_nc[b, i], dec[0], rtol=0, atol=1e-14)


def test_ragged_chunk_with_equal_lengths_is_the_batched_chunk():
    """With every past[b] equal, the ragged step is prefill_chunk of the whole batch."""
    w = synthetic.WORKLOADS["prefill_f32"]
    inp = synthetic.make_prefill(w, seq=24, batch=3)
    kc = np.full((3, 40, w.hkv, w.d), 0.5)
    vc = np.full((3, 40, w.hkv, w.d), 1.5)
    q, k, v = inp["q"][:, :10], inp["k"][:, :10], inp["v"][:, :10]
    a = oracle.prefill_chunk(q, k, v, kc, vc, 11, inp["qw"], inp["kw"], inp["cos"], inp["sin"], w.half, w.eps,
                             w.scale, True)
    r = oracle.prefill_chunk_ragged(q, k, v, kc, vc, [11, 11, 11], inp["qw"], inp["kw"], inp["cos"], inp["sin"],
                                    w.half, w.eps, w.scale, True)
    for x, y in zip(a, r):
        np.testing.assert_array_equal(x, y)


def test_tiny_workload_end_to_end_against_library_routines():
    """The tiny f32 workload: oracle prefill vs torch rms_norm + complex turn + SDPA."""
    w = synthetic.WORKLOADS["tiny_f32"]
    inp = synthetic.make_prefill(w)
    out, _ = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["qw"], inp["kw"], inp["cos"],
                            inp["sin"], w.half, w.eps, 0, w.scale, True)

    def prep(x, wt):
        n = _torch_rmsnorm(x, wt, w.eps)
        ang = np.arctan2(inp["sin"].astype(np.float64), inp["cos"].astype(np.float64))
        rad = np.hypot(inp["sin"].astype(np.float64), inp["cos"].astype(np.float64))
        z = (n[..., :w.half] + 1j * n[..., w.half:]) * (rad * np.exp(1j * ang))[None, :, None]
        return np.concatenate([z.real, z.imag], axis=-1)

    qh, kh = prep(inp["q"], inp["qw"]), prep(inp["k"], inp["kw"])
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(qh).permute(0, 2, 1, 3), torch.from_numpy(kh).permute(0, 2, 1, 3),
        torch.from_numpy(inp["v"].astype(np.float64)).permute(0, 2, 1, 3),
        attn_mask=torch.from_numpy(_bottom_right_mask(w.seq, w.seq)), scale=w.scale)
    np.testing.assert_allclose(out, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-13)


# ------------------------------------------------------------ packed rows with groups

@pytest.mark.parametrize("n,group,queries", [(11, 0, 0), (11, 4, 0), (11, 4, 6), (12, 3, 12), (9, 20, 5)])
def test_attended_rows_is_block_diagonal_sdpa(n, group, queries):
    """attentionRows' groups: torch SDPA over all n rows with an explicit block-diagonal
    boolean mask (query i sees key j iff i // group == j // group), scale 1/sqrt(head),
    after torch rms_norm + complex turn of q and k at table row r; out keeps the first
    `queries` rows."""
    heads, head, half = 2, 8, 4
    rng = np.random.default_rng(n * 100 + group * 10 + queries)
    qkv = rng.standard_normal((n, 3 * heads * head))
    qw, kw = rng.uniform(0.5, 1.5, head), rng.uniform(0.5, 1.5, head)
    cos, sin = _angles_tables(n, half, head)
    prep = dict(qw=qw, kw=kw, cos=cos, sin=sin, half=half, eps=1e-6)
    out, qh, kh = oracle.attended_rows(qkv, heads, head, group, queries, prep)

    x = qkv.reshape(n, 3, heads, head)

    def turn(y, wt):
        m = _torch_rmsnorm(y, wt, 1e-6)
        z = (m[..., :half] + 1j * m[..., half:]) * (cos + 1j * sin)[:, None, :]
        return np.concatenate([z.real, z.imag], axis=-1)

    q_ref, k_ref = turn(x[:, 0], qw), turn(x[:, 1], kw)
    np.testing.assert_allclose(qh, q_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(kh, k_ref, rtol=0, atol=1e-13)
    g = group if group else n
    idx = np.arange(n)
    mask = (idx[:, None] // g) == (idx[None, :] // g)
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q_ref).permute(1, 0, 2), torch.from_numpy(k_ref).permute(1, 0, 2),
        torch.from_numpy(x[:, 2].copy()).permute(1, 0, 2), attn_mask=torch.from_numpy(mask),
        scale=1 / math.sqrt(head)).permute(1, 0, 2).reshape(n, heads * head).numpy()
    nq = queries if queries else n
    assert out.shape == (nq, heads * head)
    np.testing.assert_allclose(out, ref[:nq], rtol=0, atol=1e-13)


# ------------------------------------------------------------ quantised KV cache coding

def test_kv_coding_worked_examples(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kv_coding.json")))
    for case in g["quantize"]:
        codes, lo, step, k = oracle.kv_quantize(np.array([case["x"]], np.float32), case["bits"])
        assert codes[0].tolist() == case["codes"], case["name"]
        assert float(lo[0]) == case["lo"] and float(step[0]) == case["step"], case["name"]
        assert int(k[0]) == case["k"], case["name"]
    for case in g["pack"]:
        got = oracle.kv_pack(np.array([case["codes"]]), case["bits"])[0]
        assert got.tolist() == case["bytes"], case["name"]
        assert oracle.kv_unpack(got[None], case["bits"], len(case["codes"]))[0].tolist() == case["codes"]


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_kv_quantize_is_the_least_error_candidate(bits):
    rng = np.random.default_rng(bits)
    x = np.concatenate([rng.standard_normal((20, 64)), rng.standard_t(3, (20, 64)) * 3.0]).astype(np.float32)
    codes, lo, step, k = oracle.kv_quantize(x, bits)
    for u in range(x.shape[0]):
        c, l0, s0, k0, err = np_quantize(x[u], bits)
        assert k[u] == k0 and lo[u] == l0 and step[u] == s0
        np.testing.assert_array_equal(codes[u], c)
        back = oracle.kv_dequantize(codes[u], lo[u], step[u])
        assert abs(((x[u] - back) ** 2).sum() - err.min()) <= 1e-12 * max(1.0, err.min())


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_kv_quantize_invariants(bits):
    rng = np.random.default_rng(10 + bits)
    x = (rng.standard_normal((50, 128)) * rng.uniform(0.1, 10, (50, 1))).astype(np.float32)
    codes, lo, step, k = oracle.kv_quantize(x, bits)
    top = 2 ** bits - 1
    assert codes.min() >= 0 and codes.max() <= top
    back = oracle.kv_dequantize(codes, lo, step)
    inside = (x >= lo[:, None]) & (x <= lo[:, None] + top * step[:, None].astype(np.float64))
    # inside the range every value comes back within half a step (plus f32 rounding)
    assert (np.abs(x - back)[inside] <= (0.5 + 1e-5) * np.broadcast_to(step[:, None], x.shape)[inside]).all()
    # scaling by a power of two scales the range exactly and keeps the codes
    c2, lo2, st2, k2 = oracle.kv_quantize(x * np.float32(8.0), bits)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(k2, k)
    np.testing.assert_array_equal(lo2, lo * np.float32(8.0))
    np.testing.assert_array_equal(st2, step * np.float32(8.0))
    # the chosen range is never worse than min..max (candidate 0 up to its f32 rounding)
    mn, mx = x.min(axis=1), x.max(axis=1)
    st0 = (mx - mn) / np.float32(top)
    c0 = np.clip(np.rint((x - mn[:, None]) * (np.float32(1) / st0)[:, None]), 0, top)
    err0 = ((x - (mn[:, None].astype(np.float64) + st0[:, None] * c0)) ** 2).sum(axis=1)
    assert (((x - back) ** 2).sum(axis=1) <= err0 * (1 + 1e-4)).all()


def test_kv_quantize_constant_head_and_fewer_bits_more_error():
    x = np.full((2, 32), 1.25, np.float32)
    codes, lo, step, _ = oracle.kv_quantize(x, 4)
    assert (codes == 0).all() and (lo == 1.25).all() and (step == 0).all()
    np.testing.assert_array_equal(oracle.kv_dequantize(codes, lo, step), x)
    y = np.random.default_rng(3).standard_normal((200, 128)).astype(np.float32)
    errs = []
    for bits in (8, 4, 2):
        c, l0, s0, _ = oracle.kv_quantize(y, bits)
        errs.append(((y - oracle.kv_dequantize(c, l0, s0)) ** 2).mean())
    assert errs[0] < errs[1] < errs[2]
    # a uniform quantiser's error on N(0, 1) is about step^2 / 12: 8 bits at ~5.5 sigma / 255
    assert 0.5 < errs[0] / ((5.5 / 255) ** 2 / 12) < 2.0


# ------------------------------------------------------------ 8-bit attention operands

def test_e4m3_rounding_is_torch_float8_e4m3fn():
    """E4M3 coding = torch's float8_e4m3fn conversion (nearest, ties to even) of x (1/s), on
    every E4M3 number, every midpoint and its neighbours, and random values, with s = 1
    (units whose largest magnitude is 448)."""
    codes = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = (codes[:-1] + codes[1:]) / 2
    xs = np.concatenate([codes, mids, np.nextafter(mids, 1e9, dtype=np.float32),
                         np.nextafter(mids, -1e9, dtype=np.float32),
                         RNG.uniform(-448, 448, 4000).astype(np.float32)]).astype(np.float32)
    xs = np.concatenate([xs, -xs])
    n = 448
    units = []
    for i in range(0, len(xs), n - 1):
        u = np.zeros(n, np.float32)
        chunk = xs[i:i + n - 1]
        u[:len(chunk)] = chunk
        u[-1] = 448.0                       # every unit's largest magnitude: scale 1
        units.append(u)
    units = np.stack(units)
    vals, scale = oracle.e4m3_code(units)
    assert (scale == 1.0).all()
    ref = torch.from_numpy(units).to(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(vals, ref)


def test_int8_coding():
    x = (RNG.standard_normal((40, 128)) * RNG.uniform(0.01, 100, (40, 1))).astype(np.float32)
    codes, scale = oracle.int8_code(x)
    amax = np.abs(x).max(axis=1)
    np.testing.assert_array_equal(scale, (amax / np.float32(127)).astype(np.float32))
    inv = (np.float32(1) / scale).astype(np.float32)
    np.testing.assert_array_equal(codes, np.clip(np.rint(x * inv[:, None]), -127, 127).astype(np.int8))
    assert np.abs(codes).max() == 127
    back = codes.astype(np.float64) * scale[:, None]
    assert (np.abs(back - x) <= 0.5 * scale[:, None] * (1 + 1e-6)).all()
    c0, s0 = oracle.int8_code(np.zeros((1, 8), np.float32))
    assert (c0 == 0).all() and s0[0] == 1.0


def test_rows8_operands_are_exact_on_exact_inputs():
    """Rows whose q and k are multiples of their unit's scale (largest magnitude 127 of them)
    and whose v lie on the E4M3 grid of their group's scale come back unchanged, so the
    8-bit attention equals the exact one; this pins the units (q per row, k per 64-key
    tile restarting at every group, v per group) and the composition."""
    n, heads, head, group = 150, 2, 16, 100
    rng = np.random.default_rng(8)
    x = np.zeros((n, 3, heads, head), np.float32)
    x[:, 0] = rng.integers(-126, 127, (n, heads, head)) * np.float32(2.0 ** -6)
    x[:, 0, :, 0] = 127 * np.float32(2.0 ** -6)                    # q: every row's max 127 s
    x[:, 1] = rng.integers(-126, 127, (n, heads, head)) * np.float32(2.0 ** -5)
    for t0 in (0, 64, 100):                                          # tiles 0-63, 64-99, 100-149
        x[t0, 1, :, 1] = 127 * np.float32(2.0 ** -5)
    grid = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    x[:, 2] = rng.choice(np.concatenate([grid, -grid]), (n, heads, head)) * np.float32(2.0 ** -4)
    x[0, 2, :, 0] = x[100, 2, :, 0] = 448 * np.float32(2.0 ** -4)    # each group's v max
    ops = oracle.rows8_operands(x.reshape(n, -1), heads, head, group)
    np.testing.assert_array_equal(ops["q_back"], x[:, 0])
    np.testing.assert_array_equal(ops["k_back"], x[:, 1])
    np.testing.assert_array_equal(ops["v_back"], x[:, 2])
    assert len(np.unique(ops["sk"][:, 0])) == 1                      # one k scale (same max)
    out8, _ = oracle.attended_rows8(ops, heads, head, group)
    ref, _, _ = oracle.attended_rows(x.reshape(n, -1), heads, head, group)
    np.testing.assert_allclose(out8, ref, rtol=0, atol=1e-13)


def test_rows8_key_tiles_restart_at_groups():
    n, heads, head, group = 150, 1, 8, 100
    rng = np.random.default_rng(9)
    x = rng.standard_normal((n, 3 * heads * head)).astype(np.float32)
    x[70, heads * head:2 * heads * head] *= 50        # a large key in tile 64..99 only
    ops = oracle.rows8_operands(x, heads, head, group)
    sk = ops["sk"][:, 0]
    assert (sk[64:100] == sk[70]).all()
    assert sk[70] > 10 * sk[0] and sk[70] > 10 * sk[100]
    assert (sk[:64] == sk[0]).all() and (sk[100:150] == sk[100]).all()
    sv = ops["sv"][:, 0]
    assert (sv[:100] == sv[0]).all() and (sv[100:] == sv[100]).all()


# ------------------------------------------------------------------- input generation

def test_bf16_rounding_matches_torch():
    x = np.concatenate([RNG.standard_normal(100000) * 10.0 ** RNG.integers(-6, 6, 100000),
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, 3.0e38])])
    got = synthetic.bf16_round(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(got, ref)


def test_workload_shapes_and_tables():
    w = synthetic.WORKLOADS["long_prefill_bf16"]
    inp = synthetic.make_prefill(w, seq=1000, batch=1)
    assert inp["q"].shape == (1, 1000, 64, 128) and inp["k"].shape == (1, 1000, 8, 128)
    assert len(inp["outliers"]) == 10
    np.testing.assert_array_equal(synthetic.bf16_round(inp["k"]), inp["k"])
    cos, sin = synthetic.rope_tables(5, 64, 128, 1e6)
    ang = 3 * 1e6 ** (-2 * 5 / 128)
    assert cos[3, 5] == np.float32(math.cos(ang)) and sin[3, 5] == np.float32(math.sin(ang))


# ----------------------------------------------------------------------- paged KV pool

def _scatter_pool(caches, lens, page_rows, num_pages, shared, rng):
    """Write each sequence's rows into pages of a pool, page by page, with a loop of its
    own: a random distinct page per (sequence, page slot), except that the first `shared`
    page slots of every sequence point at sequence 0's pages (their rows must be equal)."""
    B = caches.shape[0]
    max_pages = (caches.shape[1] + page_rows - 1) // page_rows
    free = list(rng.permutation(num_pages))
    pages = np.full((B, max_pages), -1, dtype=np.int32)
    pool = np.full((num_pages, page_rows) + caches.shape[2:], np.nan)
    for b in range(B):
        for slot in range((lens[b] + page_rows - 1) // page_rows):
            if b > 0 and slot < shared:
                pages[b, slot] = pages[0, slot]
                continue
            pages[b, slot] = free.pop()
            for r in range(page_rows):
                j = slot * page_rows + r
                if j < lens[b]:
                    pool[pages[b, slot], r] = caches[b, j]
    return pool, pages


def test_paged_rows_give_back_the_scattered_caches():
    """Gathering through the page table returns every sequence's rows exactly, with shared
    prefix pages read by several sequences from one copy."""
    rng = np.random.default_rng(41)
    B, L, P = 3, 70, 16
    caches = rng.standard_normal((B, L, 2, 8))
    caches[1:, :32] = caches[0, :32]                 # a common start of two full pages
    lens = [70, 45, 33]
    pool, pages = _scatter_pool(caches, lens, P, 20, shared=2, rng=rng)
    assert (pages[1, :2] == pages[0, :2]).all() and (pages[2, :2] == pages[0, :2]).all()
    for b in range(B):
        np.testing.assert_array_equal(oracle.paged_rows(pool, pages[b], lens[b]), caches[b, :lens[b]])
    got = oracle.gather_paged(pool, pages, lens)
    for b in range(B):
        np.testing.assert_array_equal(got[b, :lens[b]], caches[b, :lens[b]])
        assert (got[b, lens[b]:] == 0).all()


def test_decode_paged_is_decode_of_the_gathered_caches():
    """decode_paged equals decode on contiguous caches holding the same rows (and is not
    fooled by NaN rows of unused pool slots)."""
    rng = np.random.default_rng(43)
    B, L, hq, hkv, d, P = 2, 50, 4, 2, 16, 16
    k = rng.standard_normal((B, L, hkv, d))
    v = rng.standard_normal((B, L, hkv, d))
    lens = [50, 21]
    kp, pages = _scatter_pool(k, lens, P, 10, shared=0, rng=np.random.default_rng(1))
    vp, pages_v = _scatter_pool(v, lens, P, 10, shared=0, rng=np.random.default_rng(1))
    assert (pages == pages_v).all()
    q = rng.standard_normal((B, hq, d))
    qw = np.ones(d)
    cos, sin = synthetic.rope_tables(64, d // 2, d, 1e4)
    kc = np.zeros((B, L, hkv, d))
    vc = np.zeros((B, L, hkv, d))
    for b in range(B):
        kc[b, :lens[b]] = k[b, :lens[b]]
        vc[b, :lens[b]] = v[b, :lens[b]]
    ref = oracle.decode(q, kc, vc, lens, [50, 21], qw, cos, sin, d // 2, 1e-6, 0.25)
    got = oracle.decode_paged(q, kp, vp, pages, lens, [50, 21], qw, cos, sin, d // 2, 1e-6, 0.25)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    assert np.isfinite(got).all()
