"""Float64 reference forward pass of a pre-norm Llama/Qwen decoder (test infrastructure).

The pages (MegaOps abstract; "Production Megakernels" lecture summary) name the
workloads -- dense Llama-3 and Qwen3 decoders -- but never write the block out.
This module takes the plainest standard reading, one step at a time:

  xn   = RMSNorm(x; g_attn)                     eps inside the square root
  q,k,v = xn Wq^T, xn Wk^T, xn Wv^T             no biases
  (Qwen3) q_h, k_h = RMSNorm_hd(.; g_q / g_k)   per head, before RoPE
  q,k  = RoPE(., p)                             rotate-half pairs (i, i + hd/2)
  cache[p] = k, v                               stored in the cache's type
  o_h  = softmax(q_h K_g^T / sqrt(hd)) V_g      g = h // (nq / nkv)
  h    = x + concat(o) Wo^T
  a    = silu(RMSNorm(h; g_ffn) Wg^T) * (RMSNorm(h; g_ffn) Wu^T)
  x'   = h + a Wd^T
  logits = RMSNorm(x_L; g_final) W_lm^T

All arithmetic is float64 (the timed CPU baseline runs the same functions on
float32 weights).  Weights arrive as the workload's storage arrays (bf16 bit
patterns or float32) and are widened exactly.  Rotary angles are always
computed in float64.  The only rounding to
a narrower type is where the decoder itself stores into its KV cache, whose
element type is part of the model (bf16 for the bf16 models).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------- storage types

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly: the bf16 value is the top half of an fp32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_f64(arr: np.ndarray) -> np.ndarray:
    if arr.dtype == np.uint16:
        return bf16_bits_to_f64(arr)
    return arr.astype(np.float64)


def widen(arr: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Storage values (bf16 bit patterns or float32) as ``dtype`` (float64, or
    float32 for the timed CPU baseline); exact for both: a bf16 value is an
    fp32 value."""
    if arr.dtype == np.uint16:
        return (arr.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(dtype, copy=False)
    return arr.astype(dtype, copy=False)


def store_like(x: np.ndarray, like_dtype) -> np.ndarray:
    """Round float64 values into a cache's storage type.

    float32 storage: nearest float32.  bf16 storage (uint16 bit patterns): the
    value goes to float32 and then to bf16 by round-to-nearest, ties to even
    on the 16 discarded bits.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if like_dtype == np.float32:
        return f
    b = f.view(np.uint32).astype(np.uint64)
    low = b & 0xFFFF
    hi = b >> 16
    up = (low > 0x8000) | ((low == 0x8000) & ((hi & 1) == 1))
    return (hi + up.astype(np.uint64)).astype(np.uint16)


# ----------------------------------------------------------------------------- elementary ops

def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * g over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_angles(pos: int, head_dim: int, theta: float) -> np.ndarray:
    """Angles p * theta^(-2i/hd) for i < hd/2, float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / head_dim)
    return float(pos) * inv


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate pairs (i, i + hd/2) of the last axis by angle p * theta^(-2i/hd)."""
    hd = x.shape[-1]
    half = hd // 2
    ang = rope_angles(pos, hd, theta)
    c, s = np.cos(ang).astype(x.dtype), np.sin(ang).astype(x.dtype)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def softmax(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Grouped-query attention of one query position.

    q: [nq, hd]; K, V: [nkv, n, hd] (the n visible keys).  Query head h reads
    KV head h // (nq / nkv).  Returns [nq, hd].
    """
    nq, hd = q.shape
    nkv = K.shape[0]
    r = nq // nkv
    out = np.empty_like(q)
    for h in range(nq):
        g = h // r
        s = (K[g] @ q[h]) / math.sqrt(hd)
        out[h] = softmax(s) @ V[g]
    return out


# ----------------------------------------------------------------------------- split-KV (flash-decoding form)

EMPTY_MAX = -math.inf   # marker of a split that holds no key


def attention_split(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Unnormalised partial attention of r query heads over one split of keys.

    q: [r, hd]; K, V: [n, hd] with n >= 0.  Returns (o [r, hd], m [r], l [r])
    with m = max_j s_j, l = sum_j exp(s_j - m), o = sum_j exp(s_j - m) V_j.
    An empty split gives o = 0, l = 0, m = EMPTY_MAX.
    """
    r, hd = q.shape
    if K.shape[0] == 0:
        return np.zeros((r, hd)), np.full(r, EMPTY_MAX), np.zeros(r)
    s = (q @ K.T) / math.sqrt(hd)          # [r, n]
    m = np.max(s, axis=1)
    e = np.exp(s - m[:, None])
    return e @ V, m, np.sum(e, axis=1)


def combine_splits(parts: Sequence[Tuple[np.ndarray, np.ndarray, np.ndarray]]) -> np.ndarray:
    """Merge split partials (o, m, l): out = sum_s e^(m_s - m) o_s / sum_s e^(m_s - m) l_s.

    Empty splits (m_s = EMPTY_MAX) are skipped.
    """
    live = [p for p in parts if np.all(np.isfinite(p[1]))]
    m = np.max(np.stack([p[1] for p in live]), axis=0)
    num = sum(np.exp(p[1] - m)[:, None] * p[0] for p in live)
    den = sum(np.exp(p[1] - m) * p[2] for p in live)
    return num / den[:, None]


# ----------------------------------------------------------------------------- model state

@dataclass
class Layer:
    wqkv: np.ndarray
    wo: np.ndarray
    wgate: np.ndarray
    wup: np.ndarray
    wdown: np.ndarray
    attn_norm: np.ndarray
    ffn_norm: np.ndarray
    q_norm: Optional[np.ndarray] = None
    k_norm: Optional[np.ndarray] = None


@dataclass
class Model:
    cfg: object                      # workloads.ModelConfig
    layers: List[Layer]
    embed: Optional[np.ndarray] = None
    lm_head: Optional[np.ndarray] = None
    final_norm: Optional[np.ndarray] = None


def prepare_layer(raw: Dict[str, np.ndarray], dtype=np.float64) -> Layer:
    """One layer's weights widened to ``dtype``: float64 for parity; the timed
    CPU baseline runs the same functions on float32 weights."""
    return Layer(**{k: widen(v, dtype) for k, v in raw.items()})


def prepare(cfg, raw_layers: Sequence[Dict[str, np.ndarray]], raw_global: Dict[str, np.ndarray],
            dtype=np.float64) -> Model:
    return Model(cfg, [prepare_layer(r, dtype) for r in raw_layers],
                 **{k: widen(v, dtype) for k, v in raw_global.items()})


@dataclass
class Trace:
    """Per-step intermediates, indexed [layer][row]."""
    x_in: List[np.ndarray] = field(default_factory=list)      # X_l, [B, H]
    q: List[np.ndarray] = field(default_factory=list)         # after QK-norm and RoPE, [B, nq, hd]
    k: List[np.ndarray] = field(default_factory=list)         # [B, nkv, hd]
    v: List[np.ndarray] = field(default_factory=list)
    attn: List[np.ndarray] = field(default_factory=list)      # concat heads, [B, nq*hd]
    attn_branch: List[np.ndarray] = field(default_factory=list)  # attn @ Wo^T, [B, H]
    h: List[np.ndarray] = field(default_factory=list)         # x + attn_branch
    act: List[np.ndarray] = field(default_factory=list)       # SwiGLU output, [B, F]
    mlp_branch: List[np.ndarray] = field(default_factory=list)
    x_out: Optional[np.ndarray] = None                        # X_L
    logits: Optional[np.ndarray] = None                       # [B, V]


def _project_qkv(cfg, lw: Layer, xn: np.ndarray):
    nq, nkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    qkv = xn @ lw.wqkv.T
    q = qkv[..., : nq * hd].reshape(*xn.shape[:-1], nq, hd)
    k = qkv[..., nq * hd:(nq + nkv) * hd].reshape(*xn.shape[:-1], nkv, hd)
    v = qkv[..., (nq + nkv) * hd:].reshape(*xn.shape[:-1], nkv, hd)
    if cfg.qk_norm:
        q = rms_norm(q, lw.q_norm, cfg.rms_eps)
        k = rms_norm(k, lw.k_norm, cfg.rms_eps)
    return q, k, v


def _mlp(cfg, lw: Layer, h: np.ndarray):
    hn = rms_norm(h, lw.ffn_norm, cfg.rms_eps)
    a = silu(hn @ lw.wgate.T) * (hn @ lw.wup.T)
    return a, a @ lw.wdown.T


def causal_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Grouped-query attention of S consecutive positions starting at 0.

    q: [S, nq, hd]; K, V: [nkv, S, hd].  Query i of head h sees keys 0..i of
    KV head h // (nq / nkv): the score matrix of each head with the entries
    above the diagonal set to -inf, then a row softmax.  Returns [S, nq, hd].
    """
    S, nq, hd = q.shape
    r = nq // K.shape[0]
    future = np.triu(np.ones((S, S), dtype=bool), 1)        # key j > query i
    out = np.empty_like(q)
    for h in range(nq):
        g = h // r
        s = (q[:, h] @ K[g].T) / math.sqrt(hd)              # [S, S]
        s[future] = -np.inf
        out[:, h] = softmax(s) @ V[g]
    return out


@dataclass
class LayerTrace:
    """One layer's intermediates for all rows (decode) or positions (prefill)."""
    q: np.ndarray               # after QK-norm and RoPE, [B, nq, hd]
    k: np.ndarray               # [B, nkv, hd]
    v: np.ndarray
    attn: np.ndarray            # concat heads, [B, nq*hd]
    attn_branch: np.ndarray     # attn @ Wo^T, [B, H]
    h: np.ndarray               # x + attn_branch
    act: np.ndarray             # SwiGLU output, [B, F]
    mlp_branch: np.ndarray
    x_out: np.ndarray           # h + mlp_branch


def _finish_layer(cfg, lw: Layer, x, qs, ks, v, att) -> LayerTrace:
    ab = att @ lw.wo.T
    h = x + ab
    a, mb = _mlp(cfg, lw, h)
    return LayerTrace(qs, ks, v, att, ab, h, a, mb, h + mb)


def decode_layer(cfg, lw: Layer, x: np.ndarray, K: np.ndarray, V: np.ndarray,
                 ctx_lens: Sequence[int]) -> LayerTrace:
    """One decoder layer of a decode step for B rows x [B, H].

    K, V: this layer's cache [B, nkv, ctx_max, hd] in storage type; the new key
    and value of row b are written at position ctx_lens[b] (0-based) and
    attention sees positions 0..ctx_lens[b].
    """
    ft = lw.wo.dtype
    B = x.shape[0]
    q, k, v = _project_qkv(cfg, lw, rms_norm(x, lw.attn_norm, cfg.rms_eps))
    att = np.empty((B, cfg.attn_cols), dtype=ft)
    qs, ks = np.empty_like(q), np.empty_like(k)
    for b in range(B):
        p = int(ctx_lens[b])
        qs[b] = rope(q[b], p, cfg.rope_theta)
        ks[b] = rope(k[b], p, cfg.rope_theta)
        K[b, :, p] = store_like(ks[b], K.dtype)
        V[b, :, p] = store_like(v[b], V.dtype)
        att[b] = attention(qs[b], widen(K[b, :, : p + 1], ft), widen(V[b, :, : p + 1], ft)).reshape(-1)
    return _finish_layer(cfg, lw, x, qs, ks, v, att)


def prefill_layer(cfg, lw: Layer, x: np.ndarray, K: np.ndarray, V: np.ndarray, row: int = 0) -> LayerTrace:
    """One decoder layer of a causal prefill of S positions x [S, H] from position 0.

    K, V: this layer's cache [rows, nkv, ctx_max, hd]; positions 0..S-1 of cache
    row ``row`` are written, and query i attends to keys 0..i.
    """
    ft = lw.wo.dtype
    S = x.shape[0]
    q, k, v = _project_qkv(cfg, lw, rms_norm(x, lw.attn_norm, cfg.rms_eps))
    qs = np.stack([rope(q[i], i, cfg.rope_theta) for i in range(S)])
    ks = np.stack([rope(k[i], i, cfg.rope_theta) for i in range(S)])
    K[row, :, :S] = store_like(ks.transpose(1, 0, 2), K.dtype)
    V[row, :, :S] = store_like(v.transpose(1, 0, 2), V.dtype)
    att = causal_attention(qs, widen(K[row, :, :S], ft), widen(V[row, :, :S], ft)).reshape(S, -1)
    return _finish_layer(cfg, lw, x, qs, ks, v, att)


def lm_head(cfg, x: np.ndarray, final_norm: np.ndarray, w_lm: np.ndarray) -> np.ndarray:
    """Logits of the rows x [B, H]: RMSNorm(x; g_final) W_lm^T."""
    return rms_norm(x, final_norm, cfg.rms_eps) @ w_lm.T


def _append(tr: Trace, x: np.ndarray, lt: LayerTrace) -> None:
    tr.x_in.append(x)
    tr.q.append(lt.q); tr.k.append(lt.k); tr.v.append(lt.v); tr.attn.append(lt.attn)
    tr.attn_branch.append(lt.attn_branch); tr.h.append(lt.h); tr.act.append(lt.act)
    tr.mlp_branch.append(lt.mlp_branch)


def decode_step(model: Model, K: np.ndarray, V: np.ndarray, ctx_lens: Sequence[int],
                tokens: Optional[np.ndarray] = None, x0: Optional[np.ndarray] = None) -> Trace:
    """One decode step for B sequences.

    K, V: caches [L, B, nkv, ctx_max, hd] in storage type; the new key and value
    of row b are written at position ctx_lens[b] (0-based) and attention sees
    positions 0..ctx_lens[b].  The caller advances ctx_lens afterwards.
    Input rows are embedding rows of ``tokens`` or, for a model without an
    embedding, ``x0`` [B, H].
    """
    cfg = model.cfg
    ft = model.layers[0].wo.dtype
    x = model.embed[np.asarray(tokens)] if cfg.has_embed else np.asarray(x0, dtype=ft)
    tr = Trace()
    for l, lw in enumerate(model.layers):
        lt = decode_layer(cfg, lw, x, K[l], V[l], ctx_lens)
        _append(tr, x, lt)
        x = lt.x_out
    tr.x_out = x
    if cfg.has_lm_head:
        tr.logits = lm_head(cfg, x, model.final_norm, model.lm_head)
    return tr


def prefill(model: Model, K: np.ndarray, V: np.ndarray, tokens: Optional[np.ndarray] = None, row: int = 0,
            x0: Optional[np.ndarray] = None) -> Trace:
    """Causal forward over S tokens of one sequence starting at position 0.

    Writes cache positions 0..S-1 of batch row ``row``; query i attends to keys
    0..i.  Input rows are the embedding rows of ``tokens`` or, given instead,
    ``x0`` [S, H].  Logits are returned for the last position only ([1, V]).
    """
    cfg = model.cfg
    ft = model.layers[0].wo.dtype
    x = model.embed[np.asarray(tokens)] if x0 is None else np.asarray(x0, dtype=ft)
    tr = Trace()
    for l, lw in enumerate(model.layers):
        lt = prefill_layer(cfg, lw, x, K[l], V[l], row)
        _append(tr, x, lt)
        x = lt.x_out
    tr.x_out = x
    if cfg.has_lm_head:
        tr.logits = lm_head(cfg, x[-1:], model.final_norm, model.lm_head)
    return tr


def argmax_lowest(logits: np.ndarray) -> np.ndarray:
    """Index of the largest value per row; the lowest index wins a tie."""
    return np.argmax(logits, axis=-1).astype(np.int32)    # numpy returns the first maximum


def max_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| over the whole tensor (the absolute error when
    the reference is all zero).  The infinity-norm form keeps near-zero entries
    of a tensor from dominating the figure."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"shapes differ: {got.shape} vs {ref.shape}")
    if got.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (den if den > 0 else 1.0)


def max_rel_err_rows(got: np.ndarray, ref: np.ndarray) -> float:
    """The largest max_rel_err over the rows of the leading axis (one row per
    sequence, or per position): a small row is judged against its own scale,
    not against the largest row of the batch."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"shapes differ: {got.shape} vs {ref.shape}")
    return max((max_rel_err(got[b], ref[b]) for b in range(ref.shape[0])), default=0.0)
