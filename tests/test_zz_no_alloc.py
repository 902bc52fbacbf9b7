"""attn_decode_static (the decode entry point that allocates nothing) against attn_decode.

attn_decode_static keeps the split partials in the library's own device scratch instead
of a caller's workspace; with the same split count it runs the same kernels, so its
output must equal attn_decode's bit for bit.  Two calls in a row (the second smaller)
check that nothing the first call left in the scratch leaks into the second; a third
lowers the default split count to fit the scratch; an explicit split count too large for
the scratch is refused before anything is enqueued.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
import transformer_attention_headprep_amd as tah
from transformer_attention_headprep_amd import attn as A
from gpu_util import assert_close, dev, host, require_gpu

pytestmark = pytest.mark.gpu


def _prep(inp):
    half = inp["half"]
    cos = dev(inp["cos"][:, :half], "f32").contiguous() if half else None
    sin = dev(inp["sin"][:, :half], "f32").contiguous() if half else None
    return tah.HeadPrep(dev(inp["qw"], "f32"), dev(inp["kw"], "f32"), cos, sin, inp["eps"])


def _inputs(w, batch=None, cache=None, seed=None):
    inp = synthetic.make_decode(w, batch=batch, cache=cache, seed=seed)
    cap = inp["k_raw"].shape[1]
    pos = np.arange(cap)[None].repeat(inp["k_raw"].shape[0], 0)
    inp["k_cache"] = synthetic.to_storage(
        oracle.headprep(inp["k_raw"], inp["kw"], inp["cos"], inp["sin"], w.half, pos, w.eps), w.dtype)
    inp["eps"] = w.eps
    return inp


def _both(w, inp, lens, pos, splits):
    """(attn_decode_static's output, attn_decode's output with the split count the static
    call used) on the same device inputs."""
    dt = w.dtype
    q, kc, vc = dev(inp["q"], dt), dev(inp["k_cache"], dt), dev(inp["v"], dt)
    lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    pos_d = torch.tensor(pos, dtype=torch.int32, device="cuda:0")
    ml = max(int(max(lens)), 1)
    prep = _prep(inp)
    got = tah.attn_decode_static(q, kc, vc, lens_d, pos_d, ml, prep=prep, scale=w.scale, splits=splits)
    torch.cuda.synchronize()
    ref = tah.attn_decode(q, kc, vc, lens_d, pos_d, ml, prep=prep, scale=w.scale, splits=splits)
    torch.cuda.synchronize()
    return host(got), host(ref)


def test_static_decode_two_calls_match_workspace_decode():
    require_gpu()
    w = synthetic.WORKLOADS["decode_bf16"]
    # first call: the whole bf16 decode workload (32 sequences x 4096 cache rows), the
    # library's split count
    inp = _inputs(w)
    b, cap = inp["q"].shape[0], inp["k_raw"].shape[1]
    assert tah.decode_workspace_size(b, w.hq, w.hkv, w.d, cap, 0) <= tah.decode_static_scratch_bytes()
    got, ref = _both(w, inp, inp["lens"], inp["pos"], 0)
    assert np.array_equal(got, ref)
    # second call, smaller: 4 ragged sequences of a 1500-row cache, three split counts
    small = _inputs(w, batch=4, cache=1500, seed=77)
    lens = np.array([1500, 1, 700, 1337], dtype=np.int32)
    pos = np.array([1500, 3, 900, 1400], dtype=np.int32)
    for splits in (0, 3, 1):
        got, ref = _both(w, small, lens, pos, splits)
        assert np.array_equal(got, ref), "splits=%d" % splits
        assert_close(got, oracle.decode(small["q"], small["k_cache"], small["v"], lens, pos, small["qw"], small["cos"],
                                        small["sin"], w.half, w.eps, w.scale), "bf16", "static decode")


def test_static_decode_f32():
    require_gpu()
    w = synthetic.Workload("d", "decode", "f32", 3, 16, 8, 900, 128, 64, 1e4, 5)
    inp = _inputs(w)
    lens = np.array([900, 450, 17], dtype=np.int32)
    pos = np.array([900, 460, 20], dtype=np.int32)
    got, ref = _both(w, inp, lens, pos, 4)
    assert np.array_equal(got, ref)


def test_static_decode_lowers_default_splits_to_fit():
    require_gpu()
    # 127 sequences x 64 q heads (d 128, two groups of 4 kv heads): the default 2 splits
    # need 2 * 127 * 64 * 130 * 4 bytes, more than the 8 MiB scratch, so the static call
    # runs one (random operands drawn on the device; this only compares the two entry
    # points)
    b, hq, hkv, d, cap = 127, 64, 8, 128, 1024
    cap_bytes = tah.decode_static_scratch_bytes()
    default = tah.decode_default_splits(b, hq, hkv, d, cap)
    per_split = b * hq * (d + 2) * 4
    assert default * per_split > cap_bytes
    lowered = max(1, min(default, cap_bytes // per_split))
    g = torch.Generator(device="cuda:0")
    g.manual_seed(11)
    q = torch.randn(b, hq, d, device="cuda:0", generator=g).to(torch.bfloat16)
    kc = (torch.randn(b, cap, hkv, d, device="cuda:0", generator=g) * 0.3).to(torch.bfloat16)
    vc = torch.randn(b, cap, hkv, d, device="cuda:0", generator=g).to(torch.bfloat16)
    lens = torch.randint(1, cap + 1, (b,), device="cuda:0", generator=g, dtype=torch.int32)
    got = tah.attn_decode_static(q, kc, vc, lens, None, cap, scale=d ** -0.5)
    ref = tah.attn_decode(q, kc, vc, lens, None, cap, scale=d ** -0.5, splits=lowered)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_static_decode_refuses_splits_beyond_scratch():
    require_gpu()
    lib = A.load_library()
    b, hq, hkv, d, cap = 64, 64, 8, 128, 1024
    splits = 16                      # 16 * 64 * 64 * 130 * 4 bytes > 8 MiB
    assert splits * b * hq * (d + 2) * 4 > tah.decode_static_scratch_bytes()
    q = torch.zeros(b, hq, d, dtype=torch.bfloat16, device="cuda:0")
    kc = torch.zeros(b, cap, hkv, d, dtype=torch.bfloat16, device="cuda:0")
    out = torch.empty_like(q)
    lens = torch.full((b,), cap, dtype=torch.int32, device="cuda:0")
    st = lib.attn_decode_static(q.data_ptr(), kc.data_ptr(), kc.data_ptr(), out.data_ptr(), b, hq, hkv, d, cap,
                                lens.data_ptr(), None, cap, 0, None, float(d ** -0.5), splits, 1, None)
    assert st == A.ATTN_ERR_WORKSPACE
    assert b"scratch" in lib.attn_last_error()
