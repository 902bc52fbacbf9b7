"""GPU parity of decode over a paged KV pool (attn_decode_paged, attn_decode_q_paged).

* Against the oracle: decode over the caches the page table gathers out of the pool
  (oracle.decode_paged), bf16 tolerance of tests/gpu_util.py.
* Against the contiguous kernels: the same rows in a contiguous cache give the same
  output bit for bit (the paged kernels only address rows differently), for every split
  count tried, bf16 and every pair of code widths.
* Shared prefixes: sequences whose tables point at the same pages read them from one copy.
* A page id outside the pool gives NaN rows for its sequence only.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
import transformer_attention_headprep_amd as tah
from gpu_util import assert_close, dev, host, require_gpu
from kv_util import oracle_cache

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _i32(x):
    return torch.tensor(np.asarray(x), dtype=torch.int32, device=DEV)


def _page_table(lens, page_rows, num_pages, shared, seed):
    """Random distinct pages per (sequence, page slot); the first `shared` slots of every
    sequence reuse sequence 0's pages.  Unused slots hold -1 (never read)."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    max_pages = max(1, (max(lens) + page_rows - 1) // page_rows)
    free = list(rng.permutation(num_pages))
    pages = np.full((B, max_pages), -1, dtype=np.int32)
    for b in range(B):
        for slot in range((lens[b] + page_rows - 1) // page_rows):
            pages[b, slot] = pages[0, slot] if (b > 0 and slot < shared) else free.pop()
    return pages


def _fill_pool(caches, pages, lens, page_rows, num_pages, fill=np.nan):
    """Pool [num_pages, page_rows, ...] holding each sequence's rows at its pages (unused
    rows `fill`); rows of shared pages come from the first sequence that uses them."""
    pool = np.full((num_pages, page_rows) + caches.shape[2:], fill)
    written = set()
    for b in range(len(lens)):
        for j in range(lens[b]):
            pg, r = pages[b, j // page_rows], j % page_rows
            if (pg, r) in written:
                continue
            pool[pg, r] = caches[b, j]
            written.add((pg, r))
    return pool


def _decode_setup(B, L, hq, hkv, d, lens, shared, seed):
    w = synthetic.Workload("pg", "decode", "bf16", B, hq, hkv, L, d, d // 2, 1e4, seed)
    inp = synthetic.make_decode(w)
    pos = np.arange(L)[None].repeat(B, 0)
    kc = synthetic.bf16_round(oracle.headprep(inp["k_raw"], inp["kw"], inp["cos"], inp["sin"], d // 2, pos, w.eps))
    vc = np.asarray(inp["v"], np.float64).copy()
    if shared:
        kc[1:, :shared] = kc[0, :shared]           # a common start: equal rows, one copy in the pool
        vc[1:, :shared] = vc[0, :shared]
    prep = tah.HeadPrep(dev(inp["qw"], "f32"), dev(inp["kw"], "f32"), dev(inp["cos"], "f32"),
                        dev(inp["sin"], "f32"), w.eps)
    return w, inp, kc, vc, prep


@pytest.mark.parametrize("page_rows", [16, 64, 256])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_decode_paged_parity(page_rows, splits):
    require_gpu()
    B, L, hq, hkv, d = 4, 700, 16, 4, 128
    lens = [700, 1, 333, 517]
    shared = 2 * page_rows if 2 * page_rows <= 333 else 0
    w, inp, kc, vc, prep = _decode_setup(B, L, hq, hkv, d, lens, shared, seed=page_rows + splits)
    num_pages = sum((n + page_rows - 1) // page_rows for n in lens) + 3
    pages = _page_table(lens, page_rows, num_pages, shared // page_rows, seed=page_rows)
    kpool = _fill_pool(kc, pages, lens, page_rows, num_pages)
    vpool = _fill_pool(vc, pages, lens, page_rows, num_pages)
    pos = [700, 3, 400, 517]
    out = tah.attn_decode_paged(dev(inp["q"], "bf16"), dev(kpool, "bf16"), dev(vpool, "bf16"), _i32(pages),
                                _i32(lens), _i32(pos), max(lens), prep=prep, scale=w.scale, splits=splits)
    got = host(out)
    assert np.isfinite(got).all()
    ref = oracle.decode_paged(inp["q"], kpool, vpool, pages, lens, pos, inp["qw"], inp["cos"], inp["sin"], d // 2,
                              w.eps, w.scale)
    assert_close(got, ref, "bf16", "paged decode, page_rows %d, splits %d" % (page_rows, splits))
    # The same rows in a contiguous cache: the same output, bit for bit.
    kcont = np.nan_to_num(oracle.gather_paged(kpool, pages, lens))
    vcont = np.nan_to_num(oracle.gather_paged(vpool, pages, lens))
    cont = tah.attn_decode(dev(inp["q"], "bf16"), dev(kcont, "bf16"), dev(vcont, "bf16"), _i32(lens), _i32(pos),
                           max(lens), prep=prep, scale=w.scale, splits=splits)
    np.testing.assert_array_equal(got, host(cont))


def test_decode_paged_shared_prefix_equals_private_copies():
    """Two sequences on one copy of a 128-row start give the rows two private copies give."""
    require_gpu()
    B, L, hq, hkv, d, P = 2, 300, 8, 2, 64, 64
    lens = [300, 260]
    w, inp, kc, vc, prep = _decode_setup(B, L, hq, hkv, d, lens, 128, seed=5)
    pos = [300, 260]
    outs = []
    for shared in (2, 0):
        num_pages = 12
        pages = _page_table(lens, P, num_pages, shared, seed=7)
        kpool = _fill_pool(kc, pages, lens, P, num_pages)
        vpool = _fill_pool(vc, pages, lens, P, num_pages)
        if shared:
            assert (pages[1, :2] == pages[0, :2]).all()
        outs.append(host(tah.attn_decode_paged(dev(inp["q"], "bf16"), dev(kpool, "bf16"), dev(vpool, "bf16"),
                                               _i32(pages), _i32(lens), _i32(pos), 300, prep=prep, scale=w.scale)))
    np.testing.assert_array_equal(outs[0], outs[1])


@pytest.mark.parametrize("splits", [1, 2])
def test_decode_paged_bad_page_gives_nan_rows(splits):
    require_gpu()
    B, L, hq, hkv, d, P = 3, 200, 8, 2, 128, 64
    lens = [200, 150, 90]
    w, inp, kc, vc, prep = _decode_setup(B, L, hq, hkv, d, lens, 0, seed=11)
    num_pages = 12
    pages = _page_table(lens, P, num_pages, 0, seed=3)
    kpool = _fill_pool(kc, pages, lens, P, num_pages, fill=0.0)
    vpool = _fill_pool(vc, pages, lens, P, num_pages, fill=0.0)
    bad = pages.copy()
    bad[1, 1] = num_pages                         # one past the pool, in a page sequence 1 reads
    pos = [200, 150, 90]
    got = host(tah.attn_decode_paged(dev(inp["q"], "bf16"), dev(kpool, "bf16"), dev(vpool, "bf16"), _i32(bad),
                                     _i32(lens), _i32(pos), 200, prep=prep, scale=w.scale, splits=splits))
    assert np.isnan(got[1]).all()
    good = host(tah.attn_decode_paged(dev(inp["q"], "bf16"), dev(kpool, "bf16"), dev(vpool, "bf16"), _i32(pages),
                                      _i32(lens), _i32(pos), 200, prep=prep, scale=w.scale, splits=splits))
    np.testing.assert_array_equal(got[[0, 2]], good[[0, 2]])


def _quant_pool(values, pages, lens, page_rows, num_pages, bits):
    """Code a cache [B, L, hkv, d] with the oracle, then place its coded rows in pages:
    codes [num_pages, hkv, page_rows, d bits / 8], params [num_pages, hkv, page_rows, 2]."""
    packed, params, back = oracle_cache(values, bits)       # [B, hkv, L, ...]
    cp = np.zeros((num_pages, packed.shape[1], page_rows, packed.shape[3]), np.uint8)
    pp = np.zeros((num_pages, params.shape[1], page_rows, 2), np.float32)
    for b in range(len(lens)):
        for j in range(lens[b]):
            pg, r = pages[b, j // page_rows], j % page_rows
            cp[pg, :, r] = packed[b, :, j]
            pp[pg, :, r] = params[b, :, j]
    return cp, pp, packed, params, back


@pytest.mark.parametrize("kb,vb", [(8, 8), (4, 4), (4, 2)])
def test_decode_q_paged_parity(kb, vb):
    require_gpu()
    B, L, hq, hkv, d, P = 3, 520, 16, 4, 128, 64
    lens = [520, 77, 300]
    w, inp, kc, vc, prep = _decode_setup(B, L, hq, hkv, d, lens, 0, seed=kb * 10 + vb)
    num_pages = sum((n + P - 1) // P for n in lens) + 2
    pages = _page_table(lens, P, num_pages, 0, seed=kb + vb)
    kcp, kpp, kpacked, kparams, kback = _quant_pool(kc, pages, lens, P, num_pages, kb)
    vcp, vpp, vpacked, vparams, vback = _quant_pool(vc, pages, lens, P, num_pages, vb)
    pos = [520, 77, 301]
    kq = tah.QuantCache(torch.from_numpy(kcp).to(DEV), torch.from_numpy(kpp).to(DEV), kb)
    vq = tah.QuantCache(torch.from_numpy(vcp).to(DEV), torch.from_numpy(vpp).to(DEV), vb)
    for splits in (0, 1, 3):
        got = host(tah.attn_decode_q_paged(dev(inp["q"], "bf16"), kq, vq, _i32(pages), _i32(lens), _i32(pos), 520,
                                           prep=prep, scale=w.scale, splits=splits))
        qh = oracle.headprep(inp["q"][:, None], inp["qw"], inp["cos"], inp["sin"], d // 2,
                             np.asarray(pos)[:, None], w.eps)
        ref = oracle.attention(qh, kback, vback, w.scale, False, lens=np.asarray(lens))[:, 0]
        assert_close(got, ref, "bf16", "paged decode_q %d/%d splits %d" % (kb, vb, splits))
        kcont = tah.QuantCache(torch.from_numpy(kpacked).to(DEV), torch.from_numpy(kparams).to(DEV), kb)
        vcont = tah.QuantCache(torch.from_numpy(vpacked).to(DEV), torch.from_numpy(vparams).to(DEV), vb)
        cont = host(tah.attn_decode_q(dev(inp["q"], "bf16"), kcont, vcont, _i32(lens), _i32(pos), 520, prep=prep,
                                      scale=w.scale, splits=splits))
        np.testing.assert_array_equal(got, cont)


def test_kv_quantize_into_pages_then_paged_decode():
    """attn_kv_quantize codes rows straight into pool pages (a page is a cache of batch 1),
    and the paged decode over them equals the contiguous decode over the same codes."""
    require_gpu()
    B, L, hq, hkv, d, P, bits = 2, 200, 8, 2, 128, 64, 4
    lens = [200, 130]
    w, inp, kc, vc, prep = _decode_setup(B, L, hq, hkv, d, lens, 0, seed=19)
    num_pages = 8
    pages = _page_table(lens, P, num_pages, 0, seed=2)
    kpool = tah.QuantCache.empty(num_pages, hkv, P, d, bits, device=DEV)
    vpool = tah.QuantCache.empty(num_pages, hkv, P, d, bits, device=DEV)
    kcont = tah.QuantCache.empty(B, hkv, L, d, bits, device=DEV)
    vcont = tah.QuantCache.empty(B, hkv, L, d, bits, device=DEV)
    kd, vd = dev(kc, "bf16"), dev(vc, "bf16")
    tah.attn_kv_quantize(kd, kcont)
    tah.attn_kv_quantize(vd, vcont)
    for b in range(B):
        for slot in range((lens[b] + P - 1) // P):
            n = min(P, lens[b] - slot * P)
            pg = int(pages[b, slot])
            page_k = tah.QuantCache(kpool.codes[pg:pg + 1], kpool.params[pg:pg + 1], bits)
            page_v = tah.QuantCache(vpool.codes[pg:pg + 1], vpool.params[pg:pg + 1], bits)
            tah.attn_kv_quantize(kd[b:b + 1, slot * P:slot * P + n].contiguous(), page_k)
            tah.attn_kv_quantize(vd[b:b + 1, slot * P:slot * P + n].contiguous(), page_v)
    pos = [200, 130]
    got = host(tah.attn_decode_q_paged(dev(inp["q"], "bf16"), kpool, vpool, _i32(pages), _i32(lens), _i32(pos), 200,
                                       prep=prep, scale=w.scale))
    cont = host(tah.attn_decode_q(dev(inp["q"], "bf16"), kcont, vcont, _i32(lens), _i32(pos), 200, prep=prep,
                                  scale=w.scale))
    np.testing.assert_array_equal(got, cont)


def _chunk_case(B, n_past, tq, hq, hkv, d, page_rows, num_pages, seed, shared=0):
    """Contiguous caches (the first n_past rows: the oracle's prepped keys, in bf16) and the
    same rows in a pool laid out by a random page table (the first `shared` pages of
    every sequence shared with sequence 0, whose prefix rows the others then copy)."""
    L = n_past + tq
    w = synthetic.Workload("pc", "prefill", "bf16", B, hq, hkv, L, d, d // 2, 1e4, seed)
    inp = synthetic.make_prefill(w)
    cap = L + 5
    kc = np.full((B, cap, hkv, d), np.nan)
    vc = np.full((B, cap, hkv, d), np.nan)
    pos = np.arange(n_past)[None].repeat(B, 0)
    kc[:, :n_past] = synthetic.bf16_round(oracle.headprep(inp["k"][:, :n_past], inp["kw"], inp["cos"], inp["sin"],
                                                          d // 2, pos, w.eps))
    vc[:, :n_past] = inp["v"][:, :n_past]
    if shared:
        kc[1:, :shared * page_rows] = kc[0, :shared * page_rows]
        vc[1:, :shared * page_rows] = vc[0, :shared * page_rows]
    lens = [L] * B
    pages = _page_table(lens, page_rows, num_pages, shared, seed=seed)
    kpool = _fill_pool(kc, pages, [n_past] * B, page_rows, num_pages)
    vpool = _fill_pool(vc, pages, [n_past] * B, page_rows, num_pages)
    return w, inp, kc, vc, kpool, vpool, pages


@pytest.mark.parametrize("page_rows,n_past,tq", [(64, 700, 300), (256, 300, 77), (64, 0, 200), (128, 1000, 1)])
def test_prefill_chunk_paged_matches_contiguous(page_rows, n_past, tq):
    """The same chunk against the same rows, in contiguous caches and in a pool: outputs and
    appended rows equal bit for bit; rows outside the sequences' pages untouched; and the
    output within the bf16 tolerance of the oracle."""
    require_gpu()
    B, hq, hkv, d = 2, 8, 2, 128
    L = n_past + tq
    num_pages = B * ((L + page_rows - 1) // page_rows) + 3
    w, inp, kc, vc, kpool, vpool, pages = _chunk_case(B, n_past, tq, hq, hkv, d, page_rows, num_pages,
                                                      seed=page_rows + n_past)
    hp = tah.HeadPrep(dev(inp["qw"], "f32"), dev(inp["kw"], "f32"), dev(inp["cos"], "f32"), dev(inp["sin"], "f32"),
                      w.eps)
    sl = slice(n_past, None)
    q, kn, vn = dev(inp["q"][:, sl], "bf16"), dev(inp["k"][:, sl], "bf16"), dev(inp["v"][:, sl], "bf16")
    kcd, vcd = dev(kc, "bf16"), dev(vc, "bf16")
    ref_out = host(tah.attn_prefill_chunk(q, kn, vn, kcd, vcd, n_past, prep=hp, causal=True, scale=w.scale))
    kpd, vpd = dev(kpool, "bf16"), dev(vpool, "bf16")
    got = host(tah.attn_prefill_chunk_paged(q, kn, vn, kpd, vpd, _i32(pages), n_past, prep=hp, causal=True,
                                            scale=w.scale))
    np.testing.assert_array_equal(got, ref_out)
    kp_after, vp_after = host(kpd), host(vpd)
    kc_after, vc_after = host(kcd), host(vcd)
    lens = [L] * B
    np.testing.assert_array_equal(oracle.gather_paged(kp_after, pages, lens), kc_after[:, :max(L, 1)])
    np.testing.assert_array_equal(oracle.gather_paged(vp_after, pages, lens), vc_after[:, :max(L, 1)])
    used = set(int(x) for x in pages.reshape(-1) if x >= 0)
    for pg in range(num_pages):
        if pg not in used:
            assert np.isnan(kp_after[pg]).all() and np.isnan(vp_after[pg]).all(), "page %d written" % pg
    ref, _, _ = oracle.prefill_chunk(inp["q"][:, sl], inp["k"][:, sl], inp["v"][:, sl], kc, vc, n_past, inp["qw"],
                                     inp["kw"], inp["cos"], inp["sin"], d // 2, w.eps, w.scale, True)
    assert_close(got, ref, "bf16", "paged chunk")


@pytest.mark.parametrize("page_rows", [64, 128])
def test_prefill_chunk_paged_per_sequence_lengths(page_rows):
    """Sequences at different cache lengths (device int32 past, the bound 520): the pool
    gives the contiguous caches' outputs and appended rows bit for bit, writes no page a
    sequence does not own, and the output is within the bf16 tolerance of the oracle."""
    require_gpu()
    B, hq, hkv, d, tq, bound = 4, 8, 2, 128, 130, 520
    past = [0, 300, 517, 64]
    w = synthetic.Workload("pr", "prefill", "bf16", B, hq, hkv, bound + tq, d, d // 2, 1e4, 401 + page_rows)
    inp = synthetic.make_prefill(w)
    cap = bound + tq + 3
    kc = np.full((B, cap, hkv, d), np.nan)
    vc = np.full((B, cap, hkv, d), np.nan)
    for b, pb in enumerate(past):
        if pb:
            kc[b, :pb] = synthetic.bf16_round(oracle.headprep(inp["k"][b:b + 1, :pb], inp["kw"], inp["cos"],
                                                              inp["sin"], d // 2, np.arange(pb)[None], w.eps))[0]
            vc[b, :pb] = inp["v"][b, :pb]
    lens = [pb + tq for pb in past]
    num_pages = sum((L + page_rows - 1) // page_rows for L in lens) + 4
    pages = _page_table(lens, page_rows, num_pages, 0, seed=page_rows)
    kpool = _fill_pool(kc, pages, past, page_rows, num_pages)
    vpool = _fill_pool(vc, pages, past, page_rows, num_pages)
    ch = {n: np.stack([inp[n][b, pb:pb + tq] for b, pb in enumerate(past)]) for n in ("q", "k", "v")}
    hp = tah.HeadPrep(dev(inp["qw"], "f32"), dev(inp["kw"], "f32"), dev(inp["cos"], "f32"), dev(inp["sin"], "f32"),
                      w.eps)
    q, kn, vn = dev(ch["q"], "bf16"), dev(ch["k"], "bf16"), dev(ch["v"], "bf16")
    pdev = _i32(past)
    kcd, vcd = dev(kc, "bf16"), dev(vc, "bf16")
    ref_out = host(tah.attn_prefill_chunk(q, kn, vn, kcd, vcd, bound, prep=hp, causal=True, scale=w.scale, past=pdev))
    kpd, vpd = dev(kpool, "bf16"), dev(vpool, "bf16")
    got = host(tah.attn_prefill_chunk_paged(q, kn, vn, kpd, vpd, _i32(pages), bound, prep=hp, causal=True,
                                            scale=w.scale, past=pdev))
    np.testing.assert_array_equal(got, ref_out)
    kp_after, vp_after = host(kpd), host(vpd)
    kc_after, vc_after = host(kcd), host(vcd)
    for b, L in enumerate(lens):
        np.testing.assert_array_equal(oracle.gather_paged(kp_after, pages[b:b + 1], [L])[0, :L], kc_after[b, :L])
        np.testing.assert_array_equal(oracle.gather_paged(vp_after, pages[b:b + 1], [L])[0, :L], vc_after[b, :L])
    used = set(int(x) for x in pages.reshape(-1) if x >= 0)
    for pg in range(num_pages):
        if pg not in used:
            assert np.isnan(kp_after[pg]).all() and np.isnan(vp_after[pg]).all(), "page %d written" % pg
    ref, _, _ = oracle.prefill_chunk_ragged(ch["q"], ch["k"], ch["v"], kc, vc, past, inp["qw"], inp["kw"], inp["cos"],
                                            inp["sin"], d // 2, w.eps, w.scale, True)
    assert_close(got, ref, "bf16", "paged ragged chunk")


def test_prefill_chunk_paged_shared_prefix_and_bad_page():
    """Two sequences on one copy of a 128-row start, each appending into its own pages,
    give what private copies give; a page id outside the pool among the pages a chunk
    writes gives NaN rows for its sequence and writes nothing."""
    require_gpu()
    B, n_past, tq, hq, hkv, d, P = 2, 200, 100, 8, 2, 128, 64
    num_pages = 12
    w, inp, kc, vc, kpool, vpool, pages = _chunk_case(B, n_past, tq, hq, hkv, d, P, num_pages, seed=77, shared=2)
    assert (pages[1, :2] == pages[0, :2]).all()
    hp = tah.HeadPrep(dev(inp["qw"], "f32"), dev(inp["kw"], "f32"), dev(inp["cos"], "f32"), dev(inp["sin"], "f32"),
                      w.eps)
    sl = slice(n_past, None)
    q, kn, vn = dev(inp["q"][:, sl], "bf16"), dev(inp["k"][:, sl], "bf16"), dev(inp["v"][:, sl], "bf16")
    got = host(tah.attn_prefill_chunk_paged(q, kn, vn, dev(kpool, "bf16"), dev(vpool, "bf16"), _i32(pages), n_past,
                                            prep=hp, causal=True, scale=w.scale))
    ref = host(tah.attn_prefill_chunk(q, kn, vn, dev(kc, "bf16"), dev(vc, "bf16"), n_past, prep=hp, causal=True,
                                      scale=w.scale))
    np.testing.assert_array_equal(got, ref)
    bad = pages.copy()
    bad[1, 4] = num_pages + 5                      # rows 256 .. 299 of sequence 1: written by this chunk
    kpd, vpd = dev(kpool, "bf16"), dev(vpool, "bf16")
    got_bad = host(tah.attn_prefill_chunk_paged(q, kn, vn, kpd, vpd, _i32(bad), n_past, prep=hp, causal=True,
                                                scale=w.scale))
    assert np.isnan(got_bad[1]).all()
    np.testing.assert_array_equal(got_bad[0], ref[0])
    kp_after = host(kpd)
    for pg in set(range(num_pages)) - set(int(x) for x in bad.reshape(-1) if 0 <= x < num_pages):
        assert np.isnan(kp_after[pg]).all(), "page %d written" % pg
