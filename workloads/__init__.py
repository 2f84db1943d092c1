"""Seeded synthetic inputs for the W4A4 rotate / quantize / GEMM path.

This module only draws random numbers and builds input tensors; it holds none
of the method's arithmetic (no rotation, no quantization, no product).  The
oracle, the GPU tests and the benchmark all take their inputs from here, so
both sides of every parity check see the same bytes.

Recipes (all values drawn in float64, then cast to fp16 with round-to-nearest-
even; "x30" means the N(0,1) draw in that channel is multiplied by 30):

  tiny     X 16x128 ~N(0,1), channels 3 and 77 x50;   W 128x128 ~N(0,0.02)
  qproj    X 2048x4096 ~N(0,1), 8 fixed channels x30;  W 4096x4096 ~N(0,0.02)
  downproj X 4096x14336 ~N(0,1), every token spikes one uniformly drawn
           channel x40;                                W 4096x14336 ~N(0,0.02)
  decode   M in {1,4,16} rows drawn like qproj's X (same outlier channels);
           W = qproj's W
  kv       8x32x4096x128 ~N(0,1), 2 fixed head_dim indices x20
  gateup   X 8192x8192 ~N(0,1), 16 fixed channels x30; W 28672x8192 ~N(0,0.015)

The outlier patterns stand in for the two layers the rotation page measures:
fixed outlier channels (its q_proj) and a channel that changes from token to
token (its down_proj).  Standard deviations are standard deviations, not
variances.

Every config owns numpy SeedSequence(1000 + index).spawn(4): stream 0 draws
X (or the decode rows), 1 draws W, 2 places the outliers, 3 draws the KV cache.
"""
from __future__ import annotations

import numpy as np

CHUNK_ROWS = 512          # rows drawn per call; keeps float64 temporaries small

CONFIG_INDEX = {"tiny": 0, "qproj": 1, "downproj": 2, "decode": 3, "gateup": 4}


def streams(config: str) -> list[np.random.Generator]:
    """The four independent generators of one config (X, W, outliers, KV)."""
    ss = np.random.SeedSequence(1000 + CONFIG_INDEX[config])
    return [np.random.default_rng(s) for s in ss.spawn(4)]


def _normal_fp16(rng: np.random.Generator, rows: int, cols: int, std: float,
                 scale_cols=None, scale_rows_cols=None, mult: float = 1.0) -> np.ndarray:
    """rows x cols fp16 array of N(0, std^2) draws, drawn row-chunk by row-chunk.

    scale_cols: channels multiplied by `mult` in every row.
    scale_rows_cols: per-row channel index multiplied by `mult` (one per row).
    """
    out = np.empty((rows, cols), dtype=np.float16)
    for r0 in range(0, rows, CHUNK_ROWS):
        r1 = min(rows, r0 + CHUNK_ROWS)
        v = rng.standard_normal((r1 - r0, cols))
        if std != 1.0:
            v *= std
        if scale_cols is not None and len(scale_cols):
            v[:, scale_cols] *= mult
        if scale_rows_cols is not None:
            v[np.arange(r1 - r0), scale_rows_cols[r0:r1]] *= mult
        out[r0:r1] = v.astype(np.float16)
    return out


def tiny() -> dict:
    gx, gw, _, _ = streams("tiny")
    ch = np.array([3, 77])
    return dict(name="tiny", X=_normal_fp16(gx, 16, 128, 1.0, scale_cols=ch, mult=50.0),
                W=_normal_fp16(gw, 128, 128, 0.02), outlier_cols=ch, outlier_mult=50.0,
                had_blocks=(128,), act_mode="sym")


def qproj_outlier_cols() -> np.ndarray:
    _, _, go, _ = streams("qproj")
    return np.sort(go.choice(4096, 8, replace=False))


def qproj(M: int = 2048, with_w: bool = True) -> dict:
    gx, gw, _, _ = streams("qproj")
    ch = qproj_outlier_cols()
    d = dict(name="qproj", X=_normal_fp16(gx, M, 4096, 1.0, scale_cols=ch, mult=30.0),
             outlier_cols=ch, outlier_mult=30.0, had_blocks=(4096, 128), act_mode="sym")
    if with_w:
        d["W"] = qproj_weight()
    return d


def qproj_weight() -> np.ndarray:
    _, gw, _, _ = streams("qproj")
    return _normal_fp16(gw, 4096, 4096, 0.02)


def downproj(M: int = 4096, with_w: bool = True) -> dict:
    gx, gw, go, _ = streams("downproj")
    spikes = go.integers(0, 14336, M)
    d = dict(name="downproj",
             X=_normal_fp16(gx, M, 14336, 1.0, scale_rows_cols=spikes, mult=40.0),
             spike_cols=spikes, outlier_mult=40.0, had_blocks=(128,), act_mode="sym")
    if with_w:
        d["W"] = _normal_fp16(gw, 4096, 14336, 0.02)
    return d


def decode(M: int, with_w: bool = True) -> dict:
    gx, _, _, _ = streams("decode")
    ch = qproj_outlier_cols()
    d = dict(name=f"decode_m{M}", X=_normal_fp16(gx, M, 4096, 1.0, scale_cols=ch, mult=30.0),
             outlier_cols=ch, outlier_mult=30.0, had_blocks=(128,), act_mode="sym")
    if with_w:
        d["W"] = qproj_weight()
    return d


def kv(B: int = 8, H: int = 32, S: int = 4096, D: int = 128) -> dict:
    """KV cache [B, H, S, D] fp16; 2 fixed head_dim indices x20 in every head."""
    _, _, go, gk = streams("decode")
    dims = np.sort(go.choice(D, 2, replace=False))
    flat = _normal_fp16(gk, B * H * S, D, 1.0, scale_cols=dims, mult=20.0)
    return dict(name="kv", KV=flat.reshape(B, H, S, D), outlier_dims=dims, outlier_mult=20.0)


def gateup_outlier_cols() -> np.ndarray:
    _, _, go, _ = streams("gateup")
    return np.sort(go.choice(8192, 16, replace=False))


def gateup(M: int = 8192, N: int = 28672, with_w: bool = True) -> dict:
    """N < 28672 draws the first N rows of the full weight (same stream prefix)."""
    gx, gw, _, _ = streams("gateup")
    ch = gateup_outlier_cols()
    d = dict(name="gateup", X=_normal_fp16(gx, M, 8192, 1.0, scale_cols=ch, mult=30.0),
             outlier_cols=ch, outlier_mult=30.0, had_blocks=(128,), act_mode="asym")
    if with_w:
        d["W"] = _normal_fp16(gw, N, 8192, 0.015)
    return d


def exact_class(seed: int, rows: int, cols: int, lim: int = 2048,
                outlier_cols=(), outlier_val: int = 2048) -> np.ndarray:
    """Integer-valued fp16 rows in [-lim, lim] (every integer there is an fp16).

    With these inputs every partial sum of a <= 8192-point transform stays an
    integer below 2^24, so fp32 arithmetic in any order is exact.
    """
    rng = np.random.default_rng(np.random.SeedSequence(77_000 + seed))
    v = rng.integers(-lim, lim + 1, size=(rows, cols)).astype(np.float64)
    for c in outlier_cols:
        v[:, c] = np.where(rng.integers(0, 2, rows) == 0, outlier_val, -outlier_val)
    return v.astype(np.float16)


def small_random(seed: int, rows: int, cols: int, std: float = 1.0,
                 outlier_cols=(), mult: float = 1.0) -> np.ndarray:
    """Generic seeded fp16 Gaussian rows for ragged / edge-case parity tests."""
    rng = np.random.default_rng(np.random.SeedSequence(55_000 + seed))
    return _normal_fp16(rng, rows, cols, std, scale_cols=np.asarray(outlier_cols, dtype=np.int64),
                        mult=mult)


def hadamard_signs(n: int, seed: int = 0) -> np.ndarray:
    """n fp16 values, each +1.0 or -1.0 with probability 1/2: the random
    diagonal of a randomized Hadamard rotation.  The draw only; what the
    signs do is the method's business, not this module's."""
    rng = np.random.default_rng(np.random.SeedSequence(66_000 + seed))
    return np.where(rng.integers(0, 2, size=n) == 0, 1.0, -1.0).astype(np.float16)


def random_bytes(seed: int, rows: int, cols: int, lo: int = 0, hi: int = 255) -> np.ndarray:
    """rows x cols uint8 drawn uniformly from [lo, hi]: raw operand bytes
    (packed 4-bit codes, biased exponents) for tests of the products alone."""
    rng = np.random.default_rng(np.random.SeedSequence(88_000 + seed))
    return rng.integers(lo, hi + 1, size=(rows, cols)).astype(np.uint8)
