"""GPU parity of attn_rows' quantised path (Q K^T on INT8, P V on E4M3).

* The quantizing pass against the oracle's 8-bit operands: without HeadPrep every code and
  scale bit for bit; with HeadPrep (f32 on the GPU, f64 in the oracle) scales to 1e-5 and
  codes within one step, nearly all equal.
* The attention over the same operands (the oracle's, written into the workspace) against
  the oracle's exact softmax over the values they give back.  Tolerance, derived from the
  E4M3 weights the GPU multiplies V with (3 fraction bits, nearest: relative error at most
  2^-4 each; below 2^-6 an absolute error of at most 2^-10 of the largest weight 448):
      |gpu - ref| <= 2^-4 B + 2^-19 len max|v| + 2^-8 |ref| + 2^-12 max|v|,
  B = sum_j p_j |v_j| / l (the oracle's attention over |v|), len = the keys a query sees;
  the last terms cover the bf16 output rounding and f32 / matrix-core accumulation.  The
  RMS error must also stay below 0.6 2^-4 RMS(B), which a systematic slip would break.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
import transformer_attention_headprep_amd as tah
from gpu_util import dev, host, require_gpu

pytestmark = pytest.mark.gpu


def _tile_key(p):
    g, b = p // 32, p % 32
    return 32 * (b // 16) + 8 * ((b % 16) // 4) + 4 * g + (b % 4)


TILE_KEYS = np.array([_tile_key(p) for p in range(64)])


def _geometry(n, group, queries):
    nq = queries if queries else n
    G = group if 0 < group < n else n
    return nq, G, (n + G - 1) // G, (G + 63) // 64


def _pack(ops, n, heads, head, group, queries):
    """The oracle's operands in the workspace layout attn_rows8 documents."""
    total, off = tah.rows8_layout(n, heads, head, group, queries)
    nq, G, groups, T = _geometry(n, group, queries)
    ws = np.zeros(total, np.uint8)

    def put(part, arr):
        b = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        ws[off[part]:off[part] + b.size] = b

    put("q8", ops["q8"])
    put("sq", ops["sq"])
    put("k8", ops["k8"])
    sk = np.ones((groups, T, heads), np.float32)       # a tile past its group's end: scale 1
    sv = np.zeros((groups, heads), np.float32)
    v8t = np.zeros((groups, T, heads, head, 64), np.float32)
    for g in range(groups):
        g0, g1 = g * G, min(g * G + G, n)
        sv[g] = ops["sv"][g0]
        for t in range(T):
            r0 = g0 + 64 * t
            if r0 >= g1:
                continue
            sk[g, t] = ops["sk"][r0]
            rows = r0 + TILE_KEYS
            ok = rows < g1
            blk = np.zeros((64, heads, head), np.float32)
            blk[ok] = ops["v8"][rows[ok]]
            v8t[g, t] = blk.transpose(1, 2, 0)
    put("sk", sk)
    put("v8t", torch.from_numpy(v8t).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    put("sv", sv)
    return ws, off


def _unpack(ws, off, n, heads, head, group, queries):
    nq, G, groups, T = _geometry(n, group, queries)

    def get(part, dtype, shape):
        cnt = int(np.prod(shape)) * np.dtype(dtype).itemsize
        return ws[off[part]:off[part] + cnt].view(dtype).reshape(shape)

    v8t = torch.from_numpy(np.ascontiguousarray(get("v8t", np.uint8, (groups, T, heads, head, 64)))).view(
        torch.float8_e4m3fn).float().numpy()
    return dict(q8=get("q8", np.int8, (nq, heads, head)), sq=get("sq", np.float32, (nq, heads)),
                k8=get("k8", np.int8, (n, heads, head)), sk=get("sk", np.float32, (groups, T, heads)),
                v8t=v8t, sv=get("sv", np.float32, (groups, heads)))


def _inputs(n, heads, head, seed, pairs=False, scale_v=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 3, heads, head))
    x[:, 2] *= scale_v
    qkv = synthetic.bf16_round(x.reshape(n, -1))
    qw = rng.uniform(0.5, 1.5, head).astype(np.float32)
    kw = rng.uniform(0.5, 1.5, head).astype(np.float32)
    cos, sin = synthetic.rope_tables(n, head // 2, head, 1e4)
    p = dict(qw=qw, kw=kw, cos=cos, sin=sin, half=head // 2, eps=1e-6, pairs=pairs)
    hp = tah.HeadPrep(dev(qw, "f32"), dev(kw, "f32"), dev(cos, "f32"), dev(sin, "f32"), 1e-6, pairs=pairs)
    return qkv, p, hp


def _check_attention(got, ref, bound, ops, n, group, what):
    G = group if 0 < group < n else n
    vmax = np.abs(ops["v_back"]).max()
    tol = 2.0 ** -4 * bound + 2.0 ** -19 * G * vmax + 2.0 ** -8 * np.abs(ref) + 2.0 ** -12 * vmax
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), what + ": non-finite output"
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError("%s: %d of %d elements outside the bound; worst at %s: |d| %.3g > %.3g"
                             % (what, bad.sum(), err.size, i, err[i], tol[i]))
    rms_err, rms_b = np.sqrt((err ** 2).mean()), np.sqrt((bound ** 2).mean())
    assert rms_err <= 0.6 * 2.0 ** -4 * rms_b, "%s: RMS error %.3g vs bound RMS %.3g" % (what, rms_err, rms_b)


@pytest.mark.parametrize("n,heads,head,group,queries", [
    (300, 4, 128, 0, 0), (300, 3, 64, 128, 0), (257, 2, 128, 100, 150), (64, 1, 128, 64, 64), (70, 2, 64, 0, 0)])
def test_rows8_quantize_exact_without_prep(n, heads, head, group, queries):
    require_gpu()
    qkv, _, _ = _inputs(n, heads, head, seed=n + head, scale_v=3.0)
    total, off = tah.rows8_layout(n, heads, head, group, queries)
    ws = torch.zeros(total, dtype=torch.uint8, device="cuda:0")
    tah.attn_rows8_quantize(dev(qkv, "bf16"), heads, head, ws, group=group, queries=queries, prep=None)
    got = _unpack(ws.cpu().numpy(), off, n, heads, head, group, queries)
    ops = oracle.rows8_operands(qkv, heads, head, group, queries, None)
    ref, _ = _pack(ops, n, heads, head, group, queries)
    ref = _unpack(ref, off, n, heads, head, group, queries)
    for part in ("q8", "sq", "k8", "sk", "sv"):
        np.testing.assert_array_equal(got[part], ref[part], err_msg=part)
    np.testing.assert_array_equal(got["v8t"], ref["v8t"])


@pytest.mark.parametrize("pairs", [False, True])
def test_rows8_quantize_with_prep(pairs):
    require_gpu()
    n, heads, head, group = 300, 4, 128, 128
    qkv, p, hp = _inputs(n, heads, head, seed=7, pairs=pairs)
    total, off = tah.rows8_layout(n, heads, head, group, 0)
    ws = torch.zeros(total, dtype=torch.uint8, device="cuda:0")
    tah.attn_rows8_quantize(dev(qkv, "bf16"), heads, head, ws, group=group, prep=hp)
    got = _unpack(ws.cpu().numpy(), off, n, heads, head, group, 0)
    ops = oracle.rows8_operands(qkv, heads, head, group, 0, p)
    ref = _unpack(_pack(ops, n, heads, head, group, 0)[0], off, n, heads, head, group, 0)
    for part in ("sq", "sk"):
        np.testing.assert_allclose(got[part], ref[part], rtol=1e-5, err_msg=part)
    for part in ("q8", "k8"):
        d = np.abs(got[part].astype(int) - ref[part].astype(int))
        assert d.max() <= 1 and (d == 0).mean() > 0.99, part
    np.testing.assert_array_equal(got["v8t"], ref["v8t"])     # v is not prepped: exact
    np.testing.assert_array_equal(got["sv"], ref["sv"])


@pytest.mark.parametrize("n,heads,head,group,queries,scale_v", [
    (300, 4, 128, 0, 0, 1.0), (300, 3, 64, 128, 0, 5.0), (257, 2, 128, 100, 150, 1.0), (64, 1, 128, 64, 64, 0.01),
    (1000, 2, 128, 0, 0, 1.0), (130, 2, 64, 1, 0, 1.0)])
def test_rows8_attend_parity(n, heads, head, group, queries, scale_v):
    """The attention alone, on the oracle's operands."""
    require_gpu()
    qkv, p, _ = _inputs(n, heads, head, seed=3 * n + heads, scale_v=scale_v)
    ops = oracle.rows8_operands(qkv, heads, head, group, queries, p)
    ws, off = _pack(ops, n, heads, head, group, queries)
    out = tah.attn_rows8_attend(torch.from_numpy(ws).cuda(), n, heads, head, group, queries)
    ref, bound = oracle.attended_rows8(ops, heads, head, group, queries)
    _check_attention(host(out), ref, bound, ops, n, group, "rows8 attend")


def test_rows8_end_to_end_without_prep():
    require_gpu()
    n, heads, head, group = 300, 4, 128, 0
    qkv, _, _ = _inputs(n, heads, head, seed=11)
    out = tah.attn_rows8(dev(qkv, "bf16"), heads, head, group=group)
    ops = oracle.rows8_operands(qkv, heads, head, group, 0, None)
    ref, bound = oracle.attended_rows8(ops, heads, head, group, 0)
    _check_attention(host(out), ref, bound, ops, n, group, "rows8")


def test_rows8_image_model_shape_sampled():
    """4608 rows of 24 heads of 128 with FLUX.3's pairs: sampled rows against the oracle's
    attention over its own 8-bit operands (the GPU's prep rounds in f32, so a few codes may
    sit one step away: the bound gets 2 % of max|v| of slack), and close to exact attention."""
    require_gpu()
    n, heads, head = 4608, 24, 128
    qkv, p, hp = _inputs(n, heads, head, seed=37, pairs=True)
    out = host(tah.attn_rows8(dev(qkv, "bf16"), heads, head, prep=hp)).reshape(n, heads, head)
    ops = oracle.rows8_operands(qkv, heads, head, 0, 0, p)
    rng = np.random.default_rng(4)
    rows = sorted({0, 1, 127, 128, 4095, 4096, n - 1} | set(rng.integers(0, n, 16).tolist()))
    sel = np.array([(0, r, (r * 5 + j) % heads) for r in rows for j in (0, 13)], dtype=np.int64)
    ref = oracle.attention_rows(ops["q_back"][None], ops["k_back"][None], ops["v_back"][None], 1 / np.sqrt(head),
                                False, sel)
    bound = oracle.attention_rows(ops["q_back"][None], ops["k_back"][None], np.abs(ops["v_back"])[None],
                                  1 / np.sqrt(head), False, sel)
    got = out[sel[:, 1], sel[:, 2]]
    vmax = np.abs(ops["v_back"]).max()
    tol = 2.0 ** -4 * bound + 2.0 ** -19 * n * vmax + 2.0 ** -8 * np.abs(ref) + 0.02 * vmax
    assert (np.abs(got - ref) <= tol).all()
