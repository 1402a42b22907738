"""Seeded generators: weights, prompts, synthetic KV caches and hidden vectors.

Every tensor draws from its own NumPy PCG64 stream, keyed by (seed, tensor
name), so any tensor can be regenerated alone and in any order. Weights are
fp16(0.02 * N(0,1)) drawn in float32; norm gains are 1; synthetic K/V caches
are fp16(N(0,1)) and hold post-rotation keys; hidden inputs are float32 N(0,1).
"""
from __future__ import annotations

import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import DecoderConfig

_STD = np.float32(0.02)


def _rng(seed: int, name: str) -> np.random.Generator:
    key = zlib.crc32(name.encode("utf-8"))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(key,))))


def _normal_f16(seed: int, name: str, shape, scale=_STD) -> np.ndarray:
    z = _rng(seed, name).standard_normal(int(np.prod(shape)), dtype=np.float32)
    if scale != 1:
        z *= np.float32(scale)
    return z.astype(np.float16).reshape(shape)


def weight_names(cfg: DecoderConfig):
    """(name, shape) of every weight tensor; matrices are row-major [out, in]."""
    d, ffn = cfg.d_model, cfg.ffn
    out = []
    if cfg.vocab:
        out.append(("embed", (cfg.vocab, d)))
    for l in range(cfg.n_layers):
        out += [
            (f"layers.{l}.attn_norm", (d,)),
            (f"layers.{l}.wqkv", (cfg.qkv_rows, d)),      # q rows, then k rows, then v rows
            (f"layers.{l}.wo", (d, cfg.q_dim)),
            (f"layers.{l}.ffn_norm", (d,)),
            (f"layers.{l}.wgate_up", (2 * ffn, d)),       # gate rows, then up rows
            (f"layers.{l}.wdown", (d, ffn)),
        ]
    if cfg.vocab:
        out += [("final_norm", (d,)), ("lm_head", (cfg.vocab, d))]
    return out


def make_weights(cfg: DecoderConfig, seed: int = 0, threads: int = 8) -> dict:
    """All weights as fp16 NumPy arrays keyed by name (gains are exactly 1)."""
    names = weight_names(cfg)

    def one(item):
        name, shape = item
        if name.endswith("norm"):
            return name, np.ones(shape, dtype=np.float16)
        return name, _normal_f16(seed, name, shape)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        return dict(ex.map(one, names))


def make_prompt(cfg: DecoderConfig, n: int, seed: int = 1) -> np.ndarray:
    """n token ids, uniform over [0, vocab)."""
    return _rng(seed, "prompt").integers(0, cfg.vocab, size=n, dtype=np.int64).astype(np.int32)


def make_kv(cfg: DecoderConfig, length: int, seed: int = 2):
    """Synthetic post-rotation cache content: K, V fp16 N(0,1), logical layout
    [layer, position, kv_head, head_dim]."""
    shape = (cfg.n_layers, length, cfg.n_kv_heads, cfg.head_dim)
    return _normal_f16(seed, "kv.k", shape, scale=1), _normal_f16(seed, "kv.v", shape, scale=1)


def make_hidden(cfg: DecoderConfig, seed: int = 2) -> np.ndarray:
    """A float32 N(0,1) hidden vector of width d_model."""
    return _rng(seed, "hidden").standard_normal(cfg.d_model, dtype=np.float32)
