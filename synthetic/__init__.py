"""Seeded synthetic inputs for the attention path's workloads.

This module is shared by the tests, the benchmark, the oracle checks and the GPU
library's callers.  It holds no step of the method: it draws random operands,
rounds them to the storage type, and builds the rotary cos/sin tables, which the
method takes as inputs (gizml:netops reference page, Types > HeadPrep: cos and sin
are given [rows, half] F32 tensors).

Recipe (every workload):
  * generator numpy.random.Generator(PCG64(seed));
  * draw order: q, k, v ~ N(0, 1) in f64; qw, kw ~ U(0.5, 1.5); then, for the long
    prefill, the token rows of k scaled by 8 (choice without replacement);
  * f32 workloads round the draws to f32; bf16 workloads round f64 -> f32 -> bf16
    (round to nearest even).  The rounded values are the inputs of both sides;
  * rotary angle of pair i at position p: p * base ** (-2 i / d), i < half, computed in
    f64, then cos and sin rounded to f32.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    dtype: str           # "f32" or "bf16"
    batch: int
    hq: int
    hkv: int
    seq: int             # prefill: sequence length; decode: cache length per sequence
    d: int
    half: int
    base: float
    seed: int
    causal: bool = True
    eps: float = 1e-6
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "prefill", "f32", 1, 1, 1, 16, 64, 32, 1e4, 1),
    "prefill_f32": Workload("prefill_f32", "prefill", "f32", 2, 8, 8, 256, 64, 32, 1e4, 2),
    "prefill_bf16": Workload("prefill_bf16", "prefill", "bf16", 4, 32, 8, 2048, 128, 64, 1e4, 3),
    "decode_bf16": Workload("decode_bf16", "decode", "bf16", 32, 32, 8, 4096, 128, 64, 1e4, 4),
    "long_prefill_bf16": Workload("long_prefill_bf16", "prefill", "bf16", 1, 64, 8, 16384, 128,
                                  64, 1e6, 5, outlier_frac=0.01, outlier_scale=8.0),
    # chunked prefill: the last 512 of 4096 tokens against a cache holding the first 3584
    "chunk_prefill_bf16": Workload("chunk_prefill_bf16", "prefill", "bf16", 4, 32, 8, 4096, 128, 64,
                                   1e4, 6, extra={"n_past": 3584, "tq": 512}),
}


def bf16_round(x) -> np.ndarray:
    """Round to bfloat16, nearest even, through f32; returned as f32 holding bf16 values."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                       # finite inputs only: no carry out of bit 31
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(f.shape)


def to_storage(x, dtype: str) -> np.ndarray:
    """f64 draws -> the storage type's values, as an f32 array."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_round(np.asarray(x, dtype=np.float32))
    raise ValueError(dtype)


def rope_tables(rows: int, half: int, d: int, base: float):
    """cos/sin [rows, half] f32 of the angle p * base**(-2 i / d), computed in f64."""
    if half == 0:
        z = np.zeros((max(rows, 1), 0), dtype=np.float32)
        return z, z.copy()
    p = np.arange(rows, dtype=np.float64)[:, None]
    i = np.arange(half, dtype=np.float64)[None, :]
    ang = p * np.power(float(base), -2.0 * i / float(d))
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def make_prefill(w: Workload, seq: int | None = None, batch: int | None = None,
                 seed: int | None = None) -> dict:
    """Prefill operands [B, S, H, D] for workload w (sizes overridable for small cases)."""
    seq = w.seq if seq is None else seq
    batch = w.batch if batch is None else batch
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    q = rng.standard_normal((batch, seq, w.hq, w.d))
    k = rng.standard_normal((batch, seq, w.hkv, w.d))
    v = rng.standard_normal((batch, seq, w.hkv, w.d))
    qw = rng.uniform(0.5, 1.5, w.d).astype(np.float32)
    kw = rng.uniform(0.5, 1.5, w.d).astype(np.float32)
    outliers = np.zeros(0, dtype=np.int64)
    if w.outlier_frac > 0:
        n_out = int(round(w.outlier_frac * seq))
        outliers = np.sort(rng.choice(seq, size=n_out, replace=False)).astype(np.int64)
        k[:, outliers] *= w.outlier_scale
    cos, sin = rope_tables(seq, w.half, w.d, w.base)
    return dict(q=to_storage(q, w.dtype), k=to_storage(k, w.dtype), v=to_storage(v, w.dtype),
                qw=qw, kw=kw, cos=cos, sin=sin, half=w.half, eps=w.eps, pos0=0,
                scale=w.scale, causal=w.causal, dtype=w.dtype, outliers=outliers)


def make_decode(w: Workload, batch: int | None = None, cache: int | None = None,
                seed: int | None = None) -> dict:
    """Decode operands: q [B, hq, D] at position `cache`, a raw key cache and a value
    cache [B, cache, hkv, D], lens = cache.  The raw keys still have to be prepped
    (HeadPrep at positions 0 .. cache-1 with kw) by whoever builds the cache."""
    batch = w.batch if batch is None else batch
    cache = w.seq if cache is None else cache
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    q = rng.standard_normal((batch, w.hq, w.d))
    k = rng.standard_normal((batch, cache, w.hkv, w.d))
    v = rng.standard_normal((batch, cache, w.hkv, w.d))
    qw = rng.uniform(0.5, 1.5, w.d).astype(np.float32)
    kw = rng.uniform(0.5, 1.5, w.d).astype(np.float32)
    cos, sin = rope_tables(cache + 1, w.half, w.d, w.base)
    return dict(q=to_storage(q, w.dtype), k_raw=to_storage(k, w.dtype),
                v=to_storage(v, w.dtype), qw=qw, kw=kw, cos=cos, sin=sin, half=w.half,
                eps=w.eps, scale=w.scale, dtype=w.dtype,
                lens=np.full(batch, cache, dtype=np.int32),
                pos=np.full(batch, cache, dtype=np.int32))
