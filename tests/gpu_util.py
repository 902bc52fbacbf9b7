"""Helpers of the GPU parity tests: device transfer and the tolerance checks.

Tolerances (the contract the GPU path is held to against the f64 oracle):
  * f32 operands: max |gpu - oracle| <= 1e-4 per element;
  * bf16 operands: |gpu - oracle| <= 2e-2 + 1e-2 |oracle| per element.
"""
import numpy as np
import torch

F32_TOL = 1e-4
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X (gfx950)"
    return torch.device("cuda:0")


def dev(x, dtype: str):
    """numpy (f32 holding f32 or bf16 values) -> device tensor of the storage type."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to("cuda:0")


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    return float(d.max(initial=0.0)), float((d / np.maximum(np.abs(ref), 1e-30)).max(initial=0.0))


def assert_close(got, ref, dtype: str, what: str = ""):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "%s: non-finite GPU output" % what
    d = np.abs(got - ref)
    if dtype == "f32":
        bad = d > F32_TOL
    else:
        bad = d > BF16_ATOL + BF16_RTOL * np.abs(ref)
    if bad.any():
        idx = np.unravel_index(np.argmax(d), d.shape)
        raise AssertionError("%s: %d of %d elements outside tolerance; max |d| = %.3g at %s "
                             "(gpu %.6g, oracle %.6g)" % (what, int(bad.sum()), d.size, d.max(),
                                                          idx, got[idx], ref[idx]))
    return errors(got, ref)
