"""Synthetic layer workloads with the shapes of the GPTQ pages' experiments.

The pages quantize real models (OPT-175B, BLOOM-176B, LLaMA) with 128 random
2048-token C4 segments as calibration data (xuzou.cn reading card for the
GPTQ paper, section 计算设置). Neither the weights nor C4 are available here,
so seeded random arrays of the same shapes stand in for them:

* W ~ N(0, sigma^2), drawn as float32, then cast to the layer dtype.
* X has 128 x 2048 = 262144 tokens (the tiny case: 4096). Each element is
  z ~ N(0, 1) drawn as float32, times an optional per-token scale
  (LogNormal(0, 0.5)), times an outlier factor on a few chosen channels,
  then cast to the activation dtype (round to nearest even).
* Outlier channels: round(frac * d_col) channels chosen without
  replacement. The astro-blog quantization survey (section 1.3 量化误差)
  describes a small fraction of channels with very large magnitude; the
  configs place that structure on the activations.

Streams: ``SeedSequence(seed).spawn(4)`` gives the generators for
[W, outlier choice, token scales, X]. X is produced in fixed chunks of
``CHUNK`` tokens; chunk c uses ``spawn(n_chunks)[c]`` of the X stream, so any
chunk can be regenerated alone and consumers can stream the matrix.
"""

from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Iterator, Optional

import numpy as np

CHUNK = 8192  # tokens per generated activation chunk


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    d_row: int
    d_col: int
    w_dtype: str
    w_sigma: float
    n_tokens: int
    x_dtype: str
    outlier_frac: float
    outlier_factor: float
    token_scale: bool
    bits: int
    group_size: int
    damp: float = 0.01
    block: int = 128
    seed: int = 0

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


def _attn(**kw) -> LayerConfig:
    base = dict(
        name="attn_proj_4096x4096_4bit_g128",
        d_row=4096,
        d_col=4096,
        w_dtype="float16",
        w_sigma=0.02,
        n_tokens=128 * 2048,
        x_dtype="float16",
        outlier_frac=0.005,
        outlier_factor=30.0,
        token_scale=True,
        bits=4,
        group_size=128,
    )
    base.update(kw)
    return LayerConfig(**base)


CONFIGS = {
    c.name: c
    for c in [
        LayerConfig(
            name="tiny_256x256_fp32_4bit_rowwise",
            d_row=256,
            d_col=256,
            w_dtype="float32",
            w_sigma=0.02,
            n_tokens=4096,
            x_dtype="float32",
            outlier_frac=0.01,
            outlier_factor=20.0,
            token_scale=False,
            bits=4,
            group_size=-1,
        ),
        _attn(),
        _attn(name="mlp_up_11008x4096_4bit_g128", d_row=11008),
        _attn(name="mlp_down_4096x11008_4bit_g128", d_col=11008),
        _attn(name="attn_proj_4096x4096_3bit_g128", bits=3),
        _attn(name="attn_proj_4096x4096_3bit_rowwise", bits=3, group_size=-1),
        _attn(
            name="opt175b_12288x12288_3bit_g128",
            d_row=12288,
            d_col=12288,
            w_sigma=0.015,
            outlier_frac=0.001,
            outlier_factor=50.0,
            token_scale=False,
            bits=3,
        ),
        _attn(
            name="opt175b_49152x12288_3bit_g128",
            d_row=49152,
            d_col=12288,
            w_sigma=0.015,
            outlier_frac=0.001,
            outlier_factor=50.0,
            token_scale=False,
            bits=3,
        ),
    ]
}


def _streams(cfg: LayerConfig):
    return np.random.SeedSequence(cfg.seed).spawn(4)


def weights(cfg: LayerConfig, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """W [d_row, d_col] in the layer dtype. ``rows`` selects a subset."""
    rng = np.random.Generator(np.random.PCG64(_streams(cfg)[0]))
    w = rng.standard_normal((cfg.d_row, cfg.d_col), dtype=np.float32)
    w *= np.float32(cfg.w_sigma)
    w = w.astype(cfg.w_dtype)
    return w if rows is None else np.ascontiguousarray(w[rows])


def n_outliers(cfg: LayerConfig) -> int:
    return int(round(cfg.outlier_frac * cfg.d_col))


def outlier_channels(cfg: LayerConfig) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(_streams(cfg)[1]))
    return np.sort(rng.choice(cfg.d_col, n_outliers(cfg), replace=False))


def channel_factors(cfg: LayerConfig) -> np.ndarray:
    f = np.ones(cfg.d_col, dtype=np.float32)
    f[outlier_channels(cfg)] = np.float32(cfg.outlier_factor)
    return f


def token_scales(cfg: LayerConfig) -> Optional[np.ndarray]:
    if not cfg.token_scale:
        return None
    rng = np.random.Generator(np.random.PCG64(_streams(cfg)[2]))
    return rng.lognormal(0.0, 0.5, cfg.n_tokens).astype(np.float32)


def _n_chunks(cfg: LayerConfig) -> int:
    return max(1, math.ceil(cfg.n_tokens / CHUNK))


def _chunk(cfg, c, seeds, factors, tscale) -> np.ndarray:
    t0 = c * CHUNK
    t1 = min(cfg.n_tokens, t0 + CHUNK)
    rng = np.random.Generator(np.random.PCG64(seeds[c]))
    z = rng.standard_normal((t1 - t0, cfg.d_col), dtype=np.float32)
    if tscale is not None:
        z *= tscale[t0:t1, None]
    z *= factors[None, :]
    return z.astype(cfg.x_dtype)


def activation_chunks(cfg: LayerConfig, threads: int = 8) -> Iterator[np.ndarray]:
    """Yield X [n_tokens, d_col] in order, CHUNK tokens at a time."""
    n = _n_chunks(cfg)
    seeds = _streams(cfg)[3].spawn(n)
    factors = channel_factors(cfg)
    tscale = token_scales(cfg)
    if threads <= 1 or n == 1:
        for c in range(n):
            yield _chunk(cfg, c, seeds, factors, tscale)
        return
    with ThreadPoolExecutor(threads) as pool:
        window = []
        for c in range(n):
            window.append(pool.submit(_chunk, cfg, c, seeds, factors, tscale))
            if len(window) > 2 * threads:
                yield window.pop(0).result()
        for f in window:
            yield f.result()


def activations(cfg: LayerConfig, threads: int = 8) -> np.ndarray:
    """The whole X [n_tokens, d_col] (only for sizes that fit in host memory)."""
    out = np.empty((cfg.n_tokens, cfg.d_col), dtype=cfg.x_dtype)
    t = 0
    for ch in activation_chunks(cfg, threads):
        out[t : t + ch.shape[0]] = ch
        t += ch.shape[0]
    return out


def small(cfg: LayerConfig, **kw) -> LayerConfig:
    """A reduced copy of a config for quick tests (same distributions)."""
    return cfg.replace(**kw)
