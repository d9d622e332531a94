"""Seeded synthetic inputs: random-init weights, KV caches, token ids, input rows.

Every tensor is drawn from its own PCG64 stream keyed by
``SeedSequence(seed, spawn_key=(kind, layer, code))``, so any tensor can be
regenerated alone, in any order, on any thread.

Storage formats (what lands in device memory and what the oracle reads):
  * matrices of a bf16 model: ``uint16`` bf16 bit patterns, rounded from the
    fp32 draw to nearest, ties to even;
  * matrices of an fp32 model: ``float32``;
  * norm gains: ``float32`` (all ones unless ``gain_jitter`` is given);
  * KV cache: the model's storage type, shape [B, n_kv, ctx_max, head_dim],
    positions below each sequence's starting context drawn N(0, 1), the rest 0.

Matrices use the [out, in] row-major layout.  The three attention input
projections are stacked into one [(nq + 2 nkv) * hd, H] matrix, rows in the
order q heads, k heads, v heads.

This module is input preparation only; it computes nothing of the decoder.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Tuple

import numpy as np

from .configs import BF16, F32, ModelConfig, RunConfig

WEIGHT_STD = 0.02

# stream kinds
K_LAYER, K_GLOBAL, K_KV, K_TOKENS, K_X0, K_GAIN = 1, 2, 3, 4, 5, 6
# per-layer tensor codes
C_WQKV, C_WO, C_WGATE, C_WUP, C_WDOWN, C_ATTN_NORM, C_FFN_NORM, C_Q_NORM, C_K_NORM = range(9)
# global tensor codes
C_EMBED, C_LM_HEAD, C_FINAL_NORM = range(3)
# token streams
C_DECODE_TOKENS, C_PREFILL_TOKENS = range(2)


def _rng(seed: int, kind: int, layer: int, code: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(kind, layer, code))))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def _normal(g: np.random.Generator, shape, std: float) -> np.ndarray:
    x = g.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _matrix(model: ModelConfig, g: np.random.Generator, shape) -> np.ndarray:
    x = _normal(g, shape, WEIGHT_STD)
    return f32_to_bf16_bits(x) if model.dtype == BF16 else x


def _gain(n: int, seed: int, layer: int, code: int, jitter: float) -> np.ndarray:
    if jitter == 0.0:
        return np.ones(n, dtype=np.float32)
    g = _rng(seed, K_GAIN, layer, code)
    return (1.0 + _normal(g, (n,), jitter)).astype(np.float32)


def layer_weights(model: ModelConfig, seed: int, layer: int, gain_jitter: float = 0.0) -> Dict[str, np.ndarray]:
    H, F, hd = model.hidden, model.ffn, model.head_dim
    w = {
        "wqkv": _matrix(model, _rng(seed, K_LAYER, layer, C_WQKV), (model.qkv_cols, H)),
        "wo": _matrix(model, _rng(seed, K_LAYER, layer, C_WO), (H, model.attn_cols)),
        "wgate": _matrix(model, _rng(seed, K_LAYER, layer, C_WGATE), (F, H)),
        "wup": _matrix(model, _rng(seed, K_LAYER, layer, C_WUP), (F, H)),
        "wdown": _matrix(model, _rng(seed, K_LAYER, layer, C_WDOWN), (H, F)),
        "attn_norm": _gain(H, seed, layer, C_ATTN_NORM, gain_jitter),
        "ffn_norm": _gain(H, seed, layer, C_FFN_NORM, gain_jitter),
    }
    if model.qk_norm:
        w["q_norm"] = _gain(hd, seed, layer, C_Q_NORM, gain_jitter)
        w["k_norm"] = _gain(hd, seed, layer, C_K_NORM, gain_jitter)
    return w


def all_layer_weights(model: ModelConfig, seed: int, gain_jitter: float = 0.0,
                      threads: int = 8) -> List[Dict[str, np.ndarray]]:
    with ThreadPoolExecutor(max(1, threads)) as ex:
        return list(ex.map(lambda l: layer_weights(model, seed, l, gain_jitter), range(model.n_layers)))


def global_weights(model: ModelConfig, seed: int, gain_jitter: float = 0.0) -> Dict[str, np.ndarray]:
    out: Dict[str, np.ndarray] = {}
    if model.has_embed:
        out["embed"] = _matrix(model, _rng(seed, K_GLOBAL, 0, C_EMBED), (model.vocab, model.hidden))
    if model.has_lm_head:
        out["lm_head"] = _matrix(model, _rng(seed, K_GLOBAL, 0, C_LM_HEAD), (model.vocab, model.hidden))
        out["final_norm"] = _gain(model.hidden, seed, 1000, C_FINAL_NORM, gain_jitter)
    return out


def kv_cache_layer(model: ModelConfig, run: RunConfig, layer: int,
                   threads: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """K and V of one layer, [B, n_kv, ctx_max, hd] in the model's storage type.
    Row b's keys and values have streams of their own, so row b is the same
    whatever the batch (given the same seed and starting context)."""
    B, G, C, hd = run.batch, model.n_kv_heads, run.ctx_max, model.head_dim
    dt = np.uint16 if model.dtype == BF16 else np.float32
    K = np.zeros((B, G, C, hd), dtype=dt)
    V = np.zeros((B, G, C, hd), dtype=dt)
    if not run.init_cache:
        return K, V

    def fill(job):
        b, which = job
        p0 = run.ctx0[b]
        g = _rng(run.seed, K_KV, layer, (b * 2 + which))
        x = _normal(g, (G, p0, hd), 1.0)
        (K, V)[which][b, :, :p0, :] = f32_to_bf16_bits(x) if model.dtype == BF16 else x

    jobs = [(b, which) for b in range(B) for which in (0, 1)]
    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, jobs))
    else:
        for j in jobs:
            fill(j)
    return K, V


def kv_cache(model: ModelConfig, run: RunConfig, threads: int = 8) -> Tuple[np.ndarray, np.ndarray]:
    """The whole cache, [L, B, n_kv, ctx_max, hd] for K and for V."""
    B, G, C, hd = run.batch, model.n_kv_heads, run.ctx_max, model.head_dim
    dt = np.uint16 if model.dtype == BF16 else np.float32
    K = np.zeros((model.n_layers, B, G, C, hd), dtype=dt)
    V = np.zeros_like(K)

    def fill(l):
        k, v = kv_cache_layer(model, run, l)
        K[l] = k
        V[l] = v
    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, range(model.n_layers)))
    return K, V


def decode_tokens(model: ModelConfig, run: RunConfig) -> np.ndarray:
    """Teacher-forced input ids, [steps, B] int32, uniform in [0, vocab)."""
    if not model.has_embed:
        return np.zeros((run.steps, run.batch), dtype=np.int32)
    g = _rng(run.seed, K_TOKENS, 0, C_DECODE_TOKENS)
    return g.integers(0, model.vocab, size=(run.steps, run.batch), dtype=np.int64).astype(np.int32)


def prefill_tokens(model: ModelConfig, run: RunConfig) -> np.ndarray:
    g = _rng(run.seed, K_TOKENS, 0, C_PREFILL_TOKENS)
    return g.integers(0, model.vocab, size=(run.prefill_len,), dtype=np.int64).astype(np.int32)


def input_rows(model: ModelConfig, run: RunConfig) -> np.ndarray:
    """Input hidden rows for a model without an embedding: [steps, B, H] fp32, N(0, 0.02^2)."""
    g = _rng(run.seed, K_X0, 0, 0)
    return _normal(g, (run.steps, run.batch, model.hidden), WEIGHT_STD)
