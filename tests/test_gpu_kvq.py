"""GPU parity of the quantised KV cache: attn_kv_quantize against the oracle's coding
(codes and ranges bit for bit; where two candidates' squared errors lie within rounding
of each other, the GPU's choice must be a candidate, coded exactly, whose error is
within rounding of the least), and attn_decode_q against the oracle's decode over the
values an oracle-coded cache gives back (bf16 tolerance of tests/gpu_util.py).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
import transformer_attention_headprep_amd as tah
from gpu_util import assert_close, dev, host, require_gpu
from kv_util import np_candidates, oracle_cache

pytestmark = pytest.mark.gpu

BITS_PAIRS = [(8, 8), (4, 4), (4, 2), (2, 2)]


def _heads(rng, shape, dtype):
    """N(0, 1) heads with per-head scales from 1e-3 to 30 and one constant head."""
    x = rng.standard_normal(shape) * rng.choice([1e-3, 0.3, 1.0, 5.0, 30.0], size=shape[:-1] + (1,))
    x[(0,) * (len(shape) - 1)] = 0.75
    return synthetic.to_storage(x, dtype)


def _check_coding(x_units, codes_g, lo_g, st_g, bits):
    """x_units [U, d] f32 values; GPU codes [U, d], lo, step [U]."""
    codes_o, lo_o, st_o, _ = oracle.kv_quantize(x_units, bits)
    same = (lo_g == lo_o) & (st_g == st_o)
    assert same.mean() >= 0.99, "GPU and oracle ranges differ on %d of %d heads" % ((~same).sum(), same.size)
    np.testing.assert_array_equal(codes_g[same], codes_o[same])
    for u in np.nonzero(~same)[0]:
        lo, st, c, err = np_candidates(x_units[u], bits)
        k = np.nonzero((lo == lo_g[u]) & (st == st_g[u]))[0]
        assert len(k) >= 1, "unit %d: the GPU's range is no candidate" % u
        np.testing.assert_array_equal(codes_g[u], c[k[0]])
        assert err[k[0]] <= err.min() * (1 + 1e-9) + 1e-30, "unit %d: not a least-error candidate" % u


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [8, 4, 2])
def test_kv_quantize_parity(dtype, d, bits):
    require_gpu()
    B, S, H, cap, row0 = 2, 37, 3, 50, 5
    rng = np.random.default_rng(100 * bits + d)
    x = _heads(rng, (B, S, H, d), dtype)
    cache = tah.QuantCache.empty(B, H, cap, d, bits, device="cuda:0")
    cache.codes.fill_(0xAB)
    cache.params.fill_(float("nan"))
    tah.attn_kv_quantize(dev(x, dtype), cache, row0=row0)
    packed = cache.codes.cpu().numpy()
    params = cache.params.cpu().numpy()
    rows = slice(row0, row0 + S)
    codes_g = oracle.kv_unpack(packed[:, :, rows], bits, d).reshape(-1, d)
    lo_g = params[:, :, rows, 0].reshape(-1)
    st_g = params[:, :, rows, 1].reshape(-1)
    units = np.ascontiguousarray(x.transpose(0, 2, 1, 3)).reshape(-1, d).astype(np.float32)
    _check_coding(units, codes_g, lo_g, st_g, bits)
    # rows outside row0 .. row0 + S - 1 are not written
    assert (packed[:, :, :row0] == 0xAB).all() and (packed[:, :, row0 + S:] == 0xAB).all()
    assert np.isnan(params[:, :, :row0]).all() and np.isnan(params[:, :, row0 + S:]).all()


def test_kv_quantize_strided_rows():
    """Keys read out of packed qkv rows (row stride 3 heads d): only the k part is coded."""
    require_gpu()
    rng = np.random.default_rng(5)
    n, heads, d = 70, 4, 128
    qkv = synthetic.bf16_round(rng.standard_normal((1, n, 3 * heads, d)))
    t = dev(qkv, "bf16")
    cache = tah.QuantCache.empty(1, heads, n, d, 4, device="cuda:0")
    tah.attn_kv_quantize(t[:, :, heads:2 * heads], cache, row0=0)
    codes_g = oracle.kv_unpack(cache.codes.cpu().numpy(), 4, d).reshape(-1, d)
    params = cache.params.cpu().numpy()
    units = np.ascontiguousarray(qkv[:, :, heads:2 * heads].transpose(0, 2, 1, 3)).reshape(-1, d).astype(np.float32)
    _check_coding(units, codes_g, params[..., 0].reshape(-1), params[..., 1].reshape(-1), 4)


def _decode_case(B, cap, hq, hkv, d, kb, vb, lens, pos, seed, pairs=False, prep=True):
    w = synthetic.Workload("q", "decode", "bf16", B, hq, hkv, cap, d, d // 2, 1e4, seed)
    inp = synthetic.make_decode(w)
    inp["cos"], inp["sin"] = synthetic.rope_tables(max(int(np.max(pos)) + 1, cap + 1), d // 2, d, 1e4)
    kpos = np.arange(cap)[None].repeat(B, 0)
    keys = synthetic.bf16_round(oracle.headprep(inp["k_raw"], inp["kw"], inp["cos"], inp["sin"], d // 2, kpos,
                                                w.eps, pairs=pairs))
    kp, kpar, kback = oracle_cache(keys, kb)
    vp, vpar, vback = oracle_cache(inp["v"], vb)
    k = tah.QuantCache(torch.from_numpy(kp).cuda(), torch.from_numpy(kpar).cuda(), kb)
    v = tah.QuantCache(torch.from_numpy(vp).cuda(), torch.from_numpy(vpar).cuda(), vb)
    hp = tah.HeadPrep(dev(inp["qw"], "f32"), dev(inp["kw"], "f32"), dev(inp["cos"], "f32"),
                      dev(inp["sin"], "f32"), w.eps, pairs=pairs) if prep else None
    qh = oracle.headprep(inp["q"][:, None], inp["qw"], inp["cos"], inp["sin"], d // 2,
                         np.asarray(pos)[:, None], w.eps, pairs=pairs) if prep else inp["q"][:, None]
    ref = oracle.attention(qh, kback, vback, w.scale, False, lens=np.asarray(lens))[:, 0]
    return w, inp, k, v, hp, ref


@pytest.mark.parametrize("kb,vb", BITS_PAIRS)
@pytest.mark.parametrize("B,cap,hq,hkv,d", [(4, 700, 16, 4, 128), (3, 300, 8, 8, 64), (2, 1000, 32, 4, 128),
                                            (2, 260, 12, 2, 64)])
def test_decode_q_parity(kb, vb, B, cap, hq, hkv, d):
    require_gpu()
    lens = [min(n, cap) for n in ([cap, 1, 333, 0] * B)[:B]]
    pos = ([cap, 5, 333, 2] * B)[:B]
    w, inp, k, v, hp, ref = _decode_case(B, cap, hq, hkv, d, kb, vb, lens, pos, seed=cap + hq + kb)
    for splits in (0, 1, 3):
        out = tah.attn_decode_q(dev(inp["q"], "bf16"), k, v, torch.tensor(lens, dtype=torch.int32, device="cuda:0"),
                                torch.tensor(pos, dtype=torch.int32, device="cuda:0"), cap, prep=hp, scale=w.scale,
                                splits=splits)
        assert_close(host(out), ref, "bf16", "decode_q bits %d/%d splits %d" % (kb, vb, splits))


@pytest.mark.parametrize("kb,vb", [(8, 8), (4, 2)])
def test_decode_q_pairs_and_no_prep(kb, vb):
    require_gpu()
    lens, pos = [500, 17], [600, 17]
    w, inp, k, v, hp, ref = _decode_case(2, 520, 16, 4, 128, kb, vb, lens, pos, seed=9, pairs=True)
    out = tah.attn_decode_q(dev(inp["q"], "bf16"), k, v, torch.tensor(lens, dtype=torch.int32, device="cuda:0"),
                            torch.tensor(pos, dtype=torch.int32, device="cuda:0"), 520, prep=hp, scale=w.scale)
    assert_close(host(out), ref, "bf16", "pairs")
    w, inp, k, v, hp, ref = _decode_case(2, 520, 16, 4, 128, kb, vb, lens, pos, seed=10, prep=False)
    out = tah.attn_decode_q(dev(inp["q"], "bf16"), k, v, torch.tensor(lens, dtype=torch.int32, device="cuda:0"),
                            None, 520, prep=None, scale=w.scale)
    assert_close(host(out), ref, "bf16", "no prep")


@pytest.mark.parametrize("kb,vb", [(8, 8), (4, 4), (4, 2)])
def test_decode_q_workload_full(kb, vb):
    """The decode workload (32 sequences x 4096 cached rows, 32 q / 8 kv heads, d 128, query
    at position 4096) with an oracle-coded cache: every output element."""
    require_gpu()
    wd = synthetic.WORKLOADS["decode_bf16"]
    inp = synthetic.make_decode(wd)
    kpos = np.arange(wd.seq)[None].repeat(wd.batch, 0)
    keys = synthetic.bf16_round(oracle.headprep(inp["k_raw"], inp["kw"], inp["cos"], inp["sin"], wd.half, kpos, wd.eps))
    kp, kpar, kback = oracle_cache(keys, kb)
    vp, vpar, vback = oracle_cache(inp["v"], vb)
    k = tah.QuantCache(torch.from_numpy(kp).cuda(), torch.from_numpy(kpar).cuda(), kb)
    v = tah.QuantCache(torch.from_numpy(vp).cuda(), torch.from_numpy(vpar).cuda(), vb)
    hp = tah.HeadPrep(dev(inp["qw"], "f32"), dev(inp["kw"], "f32"), dev(inp["cos"], "f32"), dev(inp["sin"], "f32"),
                      wd.eps)
    out = tah.attn_decode_q(dev(inp["q"], "bf16"), k, v, torch.from_numpy(inp["lens"]).cuda(),
                            torch.from_numpy(inp["pos"]).cuda(), wd.seq, prep=hp, scale=wd.scale)
    ref = oracle.decode(inp["q"], kback, vback, inp["lens"], inp["pos"], inp["qw"], inp["cos"], inp["sin"], wd.half,
                        wd.eps, wd.scale)
    assert_close(host(out), ref, "bf16", "decode workload, bits %d/%d" % (kb, vb))


def test_quantize_then_decode_end_to_end():
    """A cache appended in three pieces by attn_kv_quantize (keys prepped by attn_prep
    first) gives attn_decode_q the output the oracle gets from its own coding."""
    require_gpu()
    B, cap, hq, hkv, d, kb, vb = 2, 400, 16, 4, 128, 4, 2
    w = synthetic.Workload("e", "decode", "bf16", B, hq, hkv, cap, d, 64, 1e4, 21)
    inp = synthetic.make_decode(w)
    hp = tah.HeadPrep(dev(inp["qw"], "f32"), dev(inp["kw"], "f32"), dev(inp["cos"], "f32"), dev(inp["sin"], "f32"),
                      w.eps)
    kraw = dev(inp["k_raw"], "bf16")
    tah.attn_prep(None, kraw, hp, pos0=0)
    k = tah.QuantCache.empty(B, hkv, cap, d, kb, device="cuda:0")
    v = tah.QuantCache.empty(B, hkv, cap, d, vb, device="cuda:0")
    vv = dev(inp["v"], "bf16")
    for lo, hi in ((0, 150), (150, 151), (151, 400)):
        tah.attn_kv_quantize(kraw[:, lo:hi].contiguous(), k, row0=lo)
        tah.attn_kv_quantize(vv[:, lo:hi].contiguous(), v, row0=lo)
    lens, pos = [400, 399], [400, 399]
    out = tah.attn_decode_q(dev(inp["q"], "bf16"), k, v, torch.tensor(lens, dtype=torch.int32, device="cuda:0"),
                            torch.tensor(pos, dtype=torch.int32, device="cuda:0"), cap, prep=hp, scale=w.scale)
    kpos = np.arange(cap)[None].repeat(B, 0)
    keys = synthetic.bf16_round(oracle.headprep(inp["k_raw"], inp["kw"], inp["cos"], inp["sin"], 64, kpos, w.eps))
    _, _, kback = oracle_cache(keys, kb)
    _, _, vback = oracle_cache(inp["v"], vb)
    ref = oracle.decode(inp["q"], kback, vback, lens, pos, inp["qw"], inp["cos"], inp["sin"], 64, w.eps, w.scale)
    assert_close(host(out), ref, "bf16", "appended cache")
