"""Seeded random-init weights: N(0, 0.02) rounded to bf16, or int4 group-64 codes.

Definition (shared by every consumer, so both sides see identical model data):

* Every tensor is filled in chunks of ``CHUNK`` elements, in row-major order of
  its canonical ``[out, in]`` shape.  Chunk ``c`` of tensor ``tid`` in layer
  ``layer`` is ``Generator(PCG64(SeedSequence([seed, layer, tid, c])))
  .standard_normal(n, float32) * float32(0.02)``.  The embedding uses
  ``layer = 65535``.
* bf16 tensors keep the round-to-nearest-even bf16 of those float32 values.
* int4 tensors (linears of an ``int4`` model) quantise the same float32 values
  per output row in groups of 64 consecutive input elements:
  ``s = bf16(max|w| / 7)`` (division in float32), ``q = clip(rint(w / s), -8, 7)``
  (``rint`` rounds half to even, division in float32), and an all-zero group
  gives ``s = 0, q = 0``.  The weight the model computes with is ``q * s``.
* Norm gains are 1.0, or ``bf16(1 + gain_std * N(0,1))`` when ``gain_std > 0``
  (a test-only variant that makes a dropped or mis-indexed gain visible).

bf16 values are carried as their raw 16-bit patterns in ``uint16`` arrays.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .configs import ModelConfig

CHUNK = 1 << 22
EMBED_LAYER = 65535
TENSOR_IDS = {"wq": 0, "wk": 1, "wv": 2, "wo": 3, "wg": 4, "wu": 5, "wd": 6,
              "embed": 0, "g_attn": 7, "g_mlp": 8, "g_final": 9}
STD = np.float32(0.02)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_chunked(seed: int, layer: int, tid: int, n: int, pool=None) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    n_chunks = (n + CHUNK - 1) // CHUNK

    def fill(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, tid, c])))
        g.standard_normal(out=out[lo:hi], dtype=np.float32)
        out[lo:hi] *= STD

    if pool is None or n_chunks == 1:
        for c in range(n_chunks):
            fill(c)
    else:
        list(pool.map(fill, range(n_chunks)))
    return out


def quantize_int4_g64(w: np.ndarray):
    """Symmetric int4 quantisation in groups of 64 along the last axis.

    Returns ``(codes int8 [..., n], scales_bits uint16 [..., n/64])``.
    """
    w = np.asarray(w, dtype=np.float32)
    assert w.shape[-1] % 64 == 0
    g = w.reshape(*w.shape[:-1], w.shape[-1] // 64, 64)
    amax = np.abs(g).max(axis=-1)
    s_bits = bf16_bits_from_f32(amax / np.float32(7.0))
    s = f32_from_bf16_bits(s_bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(g / s[..., None])
    q = np.where(s[..., None] == 0, 0, q)
    q = np.clip(q, -8, 7).astype(np.int8)
    return q.reshape(w.shape), s_bits


@dataclass
class ModelWeights:
    """Host copies of one model's data.  Linears are canonical ``[out, in]``.

    bf16 models: ``layers[l][name]`` is uint16 bf16 bits.  int4 models:
    ``layers[l][name]`` is int8 codes and ``layers[l][name + '_s']`` the uint16
    bf16 scale bits ``[out, in/64]``.  Gains are uint16 bf16 bits ``[d]``.
    """
    cfg: ModelConfig
    embed: np.ndarray
    g_final: np.ndarray
    layers: list = field(default_factory=list)


def _gain(cfg: ModelConfig, layer: int, name: str) -> np.ndarray:
    if cfg.gain_std == 0.0:
        return np.full(cfg.d_model, 0x3F80, dtype=np.uint16)  # bf16(1.0)
    g = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([cfg.seed, layer, TENSOR_IDS[name], 0])))
    v = np.float32(1.0) + np.float32(cfg.gain_std) * g.standard_normal(cfg.d_model, dtype=np.float32)
    return bf16_bits_from_f32(v)


def generate_layer(cfg: ModelConfig, layer: int, pool=None) -> dict:
    out = {}
    for name, (o, i) in cfg.linear_shapes().items():
        w = _normal_chunked(cfg.seed, layer, TENSOR_IDS[name], o * i, pool).reshape(o, i)
        if cfg.weight_fmt == "int4":
            q, s = quantize_int4_g64(w)
            out[name], out[name + "_s"] = q, s
        else:
            out[name] = bf16_bits_from_f32(w)
    out["g_attn"] = _gain(cfg, layer, "g_attn")
    out["g_mlp"] = _gain(cfg, layer, "g_mlp")
    return out


def generate_weights(cfg: ModelConfig, threads: int | None = None) -> ModelWeights:
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(threads) as pool:
        emb = _normal_chunked(cfg.seed, EMBED_LAYER, TENSOR_IDS["embed"],
                              cfg.vocab * cfg.d_model, pool)
        embed = bf16_bits_from_f32(emb).reshape(cfg.vocab, cfg.d_model)
        del emb
        layers = [generate_layer(cfg, l, pool) for l in range(cfg.n_layers)]
    return ModelWeights(cfg, embed, _gain(cfg, EMBED_LAYER, "g_final"), layers)
