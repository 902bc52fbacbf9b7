"""The entry points under HIP graph capture: the library allocates nothing, never
synchronises and enqueues only kernels on the caller's stream, so a captured step
replays the eager result.  One step -- HeadPrep of k (re-copied from the raw keys each
time, since it works in place), the bf16 prefill (fixed-shift path), the split decode
(partials + merge kernel), the paged decode, the quantised decode and the 8-bit rows
path -- is captured once and replayed several times, with eager work and
synchronisations between the replays; every replay must reproduce the eager outputs bit
for bit (the kernels are deterministic)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
import transformer_attention_headprep_amd as tah
from gpu_util import dev, require_gpu

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _setup():
    wp = synthetic.Workload("gp", "prefill", "bf16", 2, 8, 2, 300, 128, 64, 1e4, 61)
    ip = synthetic.make_prefill(wp)
    t = dict(q=dev(ip["q"], "bf16"), k_raw=dev(ip["k"], "bf16"), v=dev(ip["v"], "bf16"))
    t["k"] = t["k_raw"].clone()
    prep = tah.HeadPrep(dev(ip["qw"], "f32"), dev(ip["kw"], "f32"), dev(ip["cos"], "f32"), dev(ip["sin"], "f32"),
                        wp.eps)
    t["out_p"] = torch.empty_like(t["q"])
    # decode against a cache [2, 512, 2, 128]: contiguous, paged (64-row pages reversed), coded
    wd = synthetic.Workload("gd", "decode", "bf16", 2, 8, 2, 512, 128, 64, 1e4, 62)
    idc = synthetic.make_decode(wd)
    pos = np.arange(512)[None].repeat(2, 0)
    kc = synthetic.bf16_round(oracle.headprep(idc["k_raw"], idc["kw"], idc["cos"], idc["sin"], 64, pos, wd.eps))
    t["qd"], t["kc"], t["vc"] = dev(idc["q"], "bf16"), dev(kc, "bf16"), dev(idc["v"], "bf16")
    prep_d = tah.HeadPrep(dev(idc["qw"], "f32"), dev(idc["kw"], "f32"), dev(idc["cos"], "f32"),
                          dev(idc["sin"], "f32"), wd.eps)
    t["lens"] = torch.tensor([512, 300], dtype=torch.int32, device=DEV)
    t["pos"] = torch.tensor([512, 300], dtype=torch.int32, device=DEV)
    t["ws"] = torch.empty(tah.decode_workspace_size(2, 8, 2, 128, 512, 3), dtype=torch.uint8, device=DEV)
    t["out_d"] = torch.empty_like(t["qd"])
    perm = torch.arange(16, device=DEV).flip(0)
    t["pages"] = perm.view(2, 8).to(torch.int32).contiguous()
    kp = torch.empty(16, 64, 2, 128, dtype=torch.bfloat16, device=DEV)
    vp = torch.empty_like(kp)
    kp[perm] = t["kc"].view(16, 64, 2, 128)
    vp[perm] = t["vc"].view(16, 64, 2, 128)
    t["kp"], t["vp"] = kp, vp
    t["out_pg"] = torch.empty_like(t["qd"])
    t["kq"] = tah.QuantCache.empty(2, 2, 512, 128, 4, device=DEV)
    t["vq"] = tah.QuantCache.empty(2, 2, 512, 128, 4, device=DEV)
    tah.attn_kv_quantize(t["kc"], t["kq"])
    tah.attn_kv_quantize(t["vc"], t["vq"])
    t["ws_q"] = torch.empty(tah.decode_workspace_size(2, 8, 2, 128, 512, 2), dtype=torch.uint8, device=DEV)
    t["out_q"] = torch.empty_like(t["qd"])
    # packed rows for the 8-bit path
    rng = np.random.default_rng(63)
    t["qkv"] = dev(synthetic.bf16_round(rng.standard_normal((260, 3 * 2 * 128))), "bf16")
    total, _ = tah.rows8_layout(260, 2, 128, 0, 0)
    t["ws8"] = torch.empty(total, dtype=torch.uint8, device=DEV)
    t["out8"] = torch.empty(260, 256, dtype=torch.bfloat16, device=DEV)
    return wp, wd, t, prep, prep_d


def _step(wp, wd, t, prep, prep_d):
    t["k"].copy_(t["k_raw"])
    tah.attn_prefill(t["q"], t["k"], t["v"], t["out_p"], prep=prep, causal=True, scale=wp.scale)
    tah.attn_decode(t["qd"], t["kc"], t["vc"], t["lens"], t["pos"], 512, prep=prep_d, scale=wd.scale, splits=3,
                    workspace=t["ws"], out=t["out_d"])
    tah.attn_decode_paged(t["qd"], t["kp"], t["vp"], t["pages"], t["lens"], t["pos"], 512, prep=prep_d,
                          scale=wd.scale, splits=1, out=t["out_pg"])
    tah.attn_decode_q(t["qd"], t["kq"], t["vq"], t["lens"], t["pos"], 512, prep=prep_d, scale=wd.scale, splits=2,
                      workspace=t["ws_q"], out=t["out_q"])
    tah.attn_rows8(t["qkv"], 2, 128, workspace=t["ws8"], out=t["out8"])


OUTS = ("k", "out_p", "out_d", "out_pg", "out_q", "out8")


def test_captured_step_replays_the_eager_outputs():
    require_gpu()
    wp, wd, t, prep, prep_d = _setup()
    _step(wp, wd, t, prep, prep_d)
    torch.cuda.synchronize()
    ref = {n: t[n].clone() for n in OUTS}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                  # warm the side stream as torch's capture wants
        _step(wp, wd, t, prep, prep_d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(wp, wd, t, prep, prep_d)
    scratch = torch.randn(1 << 20, device=DEV)
    for rep in range(4):
        for n in OUTS:                             # outputs scribbled over between replays
            t[n].zero_() if t[n].dtype != torch.bfloat16 else t[n].fill_(float("nan"))
        scratch.mul_(1.0001)                        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in OUTS:
            assert torch.equal(t[n].view(torch.uint8) if t[n].dtype == torch.bfloat16 else t[n],
                               ref[n].view(torch.uint8) if ref[n].dtype == torch.bfloat16 else ref[n]), \
                "replay %d: %s differs from the eager result" % (rep, n)
