"""Helpers of the quantised-cache tests: the 24 candidate ranges of a head written in
numpy float32 (vectorised, apart from the oracle's C loops), and the head-major cache
layout built from oracle-coded values."""
import numpy as np

import oracle


def np_candidates(x, bits):
    """All 24 candidates of one head x [d] (f32): lo [24], step [24], codes [24, d] and the
    f64 squared error [24] of each, each step in f32 as the coding defines it."""
    x = np.asarray(x, np.float32)
    top = np.float32(2 ** bits - 1)
    mn, mx = x.min(), x.max()
    centre = (mn + mx) * np.float32(0.5)
    r = (mx - mn) * np.float32(0.5)
    f = (np.float32(32) - np.arange(24, dtype=np.float32)) / np.float32(32)
    hw = r * f
    lo = centre - hw
    st = (hw + hw) / top
    with np.errstate(divide="ignore"):
        inv = np.float32(1) / st
    c = np.clip(np.rint((x[None, :] - lo[:, None]) * inv[:, None]), 0, top)
    back = lo[:, None].astype(np.float64) + st[:, None].astype(np.float64) * c
    err = ((x[None, :].astype(np.float64) - back) ** 2).sum(axis=1)
    return lo, st, c.astype(np.int32), err


def np_quantize(x, bits):
    """The least-error candidate of one head: codes, lo, step, k, errors of all candidates."""
    lo, st, c, err = np_candidates(x, bits)
    k = int(np.argmin(err))
    return c[k], lo[k], st[k], k, err


def oracle_cache(values, bits):
    """Code a cache of values [B, capacity, hkv, d] (f32 values) with the oracle.  Returns
    (packed codes [B, hkv, capacity, d bits / 8] uint8, params [B, hkv, capacity, 2] f32,
    the values it gives back [B, capacity, hkv, d] f64)."""
    v = np.ascontiguousarray(np.asarray(values, np.float32).transpose(0, 2, 1, 3))
    codes, lo, step, _ = oracle.kv_quantize(v, bits)
    packed = oracle.kv_pack(codes, bits)
    params = np.stack([lo, step], axis=-1).astype(np.float32)
    back = oracle.kv_dequantize(codes, lo, step).transpose(0, 2, 1, 3)
    return packed, params, np.ascontiguousarray(back)
