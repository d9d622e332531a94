"""Pins of the float64 oracle against things other than its own formulas:
brute-force scalar loops on tiny inputs, closed forms, invariants, special
cases that reduce to textbook routines, and library conversions."""
import math

import numpy as np
import pytest
import torch

from oracle import numerics as N
from workloads import ModelConfig, RunConfig, gen, BF16, F32


def rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------- storage types

def test_bf16_widening_matches_torch():
    x = torch.randn(4096, dtype=torch.float32) * 3
    bits = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want = x.to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(N.bf16_bits_to_f64(bits), want)


def test_store_bf16_round_to_nearest_even_cases():
    # 1 + 2^-8 sits half way between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    # 1 + 3 * 2^-8 sits half way between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5])
    got = N.store_like(vals, np.uint16)
    assert list(got) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020]


def test_store_bf16_matches_torch_rounding():
    x = (torch.randn(1 << 16, dtype=torch.float32) * 10)
    want = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = N.store_like(x.numpy().astype(np.float64), np.uint16)
    assert np.array_equal(got, want)


# ----------------------------------------------------------------------------- RMSNorm (P4)

def test_rmsnorm_closed_form_mean_square():
    x = rng(1).standard_normal((5, 257)) * 0.03
    eps = 1e-5
    y = N.rms_norm(x, np.ones(257), eps)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-12)


def test_rmsnorm_scale_invariant_without_eps_and_gain_elementwise():
    x = rng(2).standard_normal(64)
    g = rng(3).standard_normal(64)
    assert np.allclose(N.rms_norm(x, np.ones(64), 0.0), N.rms_norm(7.5 * x, np.ones(64), 0.0), rtol=1e-13)
    assert np.allclose(N.rms_norm(x, g, 1e-6), N.rms_norm(x, np.ones(64), 1e-6) * g, rtol=1e-13)
    # a constant row of value c normalises to sign(c) * sqrt(c^2 / (c^2 + eps))
    c = 0.01
    y = N.rms_norm(np.full(8, c), np.ones(8), 1e-5)
    assert np.allclose(y, c / math.sqrt(c * c + 1e-5), rtol=1e-14)


# ----------------------------------------------------------------------------- RoPE (P3)

@pytest.mark.parametrize("hd", [64, 128])
def test_rope_unit_vectors_closed_form(hd):
    theta, p = 5e5, 1234
    for i in (0, 1, hd // 4, hd // 2 - 1):
        e = np.zeros(hd)
        e[i] = 1.0
        y = N.rope(e, p, theta)
        ang = p * theta ** (-2.0 * i / hd)
        want = np.zeros(hd)
        want[i] = math.cos(ang)
        want[i + hd // 2] = math.sin(ang)
        assert np.allclose(y, want, atol=1e-15)
        e2 = np.zeros(hd)
        e2[i + hd // 2] = 1.0
        y2 = N.rope(e2, p, theta)
        want2 = np.zeros(hd)
        want2[i] = -math.sin(ang)
        want2[i + hd // 2] = math.cos(ang)
        assert np.allclose(y2, want2, atol=1e-15)


def test_rope_identity_at_zero_and_norm_preserving():
    x = rng(4).standard_normal((3, 128))
    assert np.array_equal(N.rope(x, 0, 1e4), x)
    for p in (1, 17, 4096, 8704):
        y = N.rope(x, p, 1e6)
        assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)


def test_rope_relative_position():
    q, k = rng(5).standard_normal(64), rng(6).standard_normal(64)
    for m, n in ((10, 3), (8000, 7999), (300, 0), (5000, 1234)):
        a = np.dot(N.rope(q, m, 1e4), N.rope(k, n, 1e4))
        b = np.dot(N.rope(q, m - n, 1e4), k)
        assert abs(a - b) < 1e-10 * max(1.0, abs(a))


# ----------------------------------------------------------------------------- softmax / attention (P1, P2, P6)

def test_softmax_rows_sum_to_one_long_context():
    for n in (1, 2, 129, 4096, 8448):
        s = rng(n).standard_normal((4, n)) * 30
        a = N.softmax(s)
        assert np.all(a >= 0)
        assert np.allclose(a.sum(axis=1), 1.0, atol=1e-12)


def brute_attention(q, K, V):
    """Scalar loops: q [nq][hd], K/V [nkv][n][hd]; query head h reads KV head h // (nq/nkv)."""
    nq, hd = len(q), len(q[0])
    nkv, n = len(K), len(K[0])
    r = nq // nkv
    out = []
    for h in range(nq):
        g = h // r
        scores = [sum(q[h][d] * K[g][j][d] for d in range(hd)) / math.sqrt(hd) for j in range(n)]
        mx = max(scores)
        w = [math.exp(s - mx) for s in scores]
        tot = sum(w)
        out.append([sum(w[j] * V[g][j][d] for j in range(n)) / tot for d in range(hd)])
    return np.array(out)


@pytest.mark.parametrize("nq,nkv,n,hd", [(4, 2, 1, 8), (4, 2, 8, 8), (2, 2, 5, 4), (8, 1, 7, 6)])
def test_attention_matches_brute_force(nq, nkv, n, hd):
    r = rng(nq * 100 + n)
    q = r.standard_normal((nq, hd))
    K = r.standard_normal((nkv, n, hd)) * 2
    V = r.standard_normal((nkv, n, hd))
    assert np.allclose(N.attention(q, K, V), brute_attention(q.tolist(), K.tolist(), V.tolist()), rtol=1e-12, atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv_and_maps_contiguous_groups():
    r = rng(9)
    q = r.standard_normal((8, 16))
    K = r.standard_normal((2, 11, 16))
    V = r.standard_normal((2, 11, 16))
    rep = 4
    Kr, Vr = np.repeat(K, rep, axis=0), np.repeat(V, rep, axis=0)
    assert np.allclose(N.attention(q, K, V), N.attention(q, Kr, Vr), rtol=1e-14)
    V2 = V.copy()
    V2[1] += 1.0                       # only heads 4..7 read KV head 1
    d = np.abs(N.attention(q, K, V2) - N.attention(q, K, V)).max(axis=1)
    assert np.all(d[:4] == 0) and np.all(d[4:] > 0.5)


def test_single_key_attention_returns_value():
    q = rng(10).standard_normal((4, 8))
    K = rng(11).standard_normal((2, 1, 8))
    V = rng(12).standard_normal((2, 1, 8))
    out = N.attention(q, K, V)
    assert np.allclose(out[:2], V[0, 0]) and np.allclose(out[2:], V[1, 0])


# ----------------------------------------------------------------------------- split-KV (P5)

@pytest.mark.parametrize("n", [1, 33, 257, 1000])
def test_split_attention_independent_of_splits(n):
    r = rng(n)
    q = r.standard_normal((4, 64))
    K = r.standard_normal((n, 64))
    V = r.standard_normal((n, 64))
    ref = N.attention(q, K[None], V[None])
    for kb in (1, 7, 32, 256, n, 4096):
        parts = [N.attention_split(q, K[s:s + kb], V[s:s + kb]) for s in range(0, max(n, 1), kb)]
        parts.append(N.attention_split(q, K[:0], V[:0]))          # an empty split is skipped
        assert np.allclose(N.combine_splits(parts), ref, rtol=1e-12, atol=1e-14)


def test_empty_split_marker():
    o, m, l = N.attention_split(np.ones((2, 4)), np.zeros((0, 4)), np.zeros((0, 4)))
    assert np.all(o == 0) and np.all(l == 0) and np.all(m == N.EMPTY_MAX)


# ----------------------------------------------------------------------------- SiLU (P8)

def test_silu_properties():
    assert N.silu(np.array([0.0]))[0] == 0.0
    assert abs(N.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(N.silu(np.array([-40.0]))[0]) < 1e-15
    for x in (-3.0, -0.5, 0.25, 2.0, 7.0):
        assert abs(N.silu(np.array([x]))[0] - x / (1.0 + math.exp(-x))) < 1e-15
        sig = 0.5 * (1.0 + math.tanh(x / 2.0))          # logistic via tanh
        assert abs(N.silu(np.array([x]))[0] - x * sig) < 1e-14


# ----------------------------------------------------------------------------- whole layer (P9, P10)

TINY = ModelConfig(name="tiny", n_layers=2, hidden=8, n_q_heads=2, n_kv_heads=1, head_dim=4,
                   ffn=12, vocab=11, rms_eps=1e-5, rope_theta=100.0, dtype=F32)
TINY_QK = ModelConfig(name="tiny-qk", n_layers=1, hidden=8, n_q_heads=4, n_kv_heads=2, head_dim=4,
                      ffn=6, vocab=13, rms_eps=1e-6, rope_theta=1e4, qk_norm=True, dtype=BF16)


def brute_layer(cfg, w, x, Kc, Vc, p):
    """One decoder layer for one row in scalar Python; Kc/Vc: lists [nkv][p][hd] of past keys."""
    H, hd, nq, nkv, F = cfg.hidden, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.ffn
    eps = cfg.rms_eps

    def norm(v, g):
        s = math.sqrt(sum(t * t for t in v) / len(v) + eps)
        return [v[i] / s * g[i] for i in range(len(v))]

    def mv(W, v):
        return [sum(W[o][i] * v[i] for i in range(len(v))) for o in range(len(W))]

    def rot(v):
        half = hd // 2
        out = [0.0] * hd
        for i in range(half):
            a = p * cfg.rope_theta ** (-2.0 * i / hd)
            out[i] = v[i] * math.cos(a) - v[i + half] * math.sin(a)
            out[i + half] = v[i + half] * math.cos(a) + v[i] * math.sin(a)
        return out

    xn = norm(x, w["attn_norm"])
    qkv = mv(w["wqkv"], xn)
    q = [qkv[h * hd:(h + 1) * hd] for h in range(nq)]
    k = [qkv[nq * hd + g * hd: nq * hd + (g + 1) * hd] for g in range(nkv)]
    v = [qkv[(nq + nkv) * hd + g * hd: (nq + nkv) * hd + (g + 1) * hd] for g in range(nkv)]
    if cfg.qk_norm:
        q = [norm(t, w["q_norm"]) for t in q]
        k = [norm(t, w["k_norm"]) for t in k]
    q = [rot(t) for t in q]
    k = [rot(t) for t in k]
    # the new key and value are read back from the cache, i.e. in its storage type
    sto = torch.bfloat16 if cfg.dtype == BF16 else torch.float32
    stored = lambda t: torch.tensor(t, dtype=torch.float64).to(sto).to(torch.float64).tolist()
    Kall = [Kc[g] + [stored(k[g])] for g in range(nkv)]
    Vall = [Vc[g] + [stored(v[g])] for g in range(nkv)]
    att = brute_attention(q, Kall, Vall).reshape(-1).tolist()
    h = [x[i] + sum(w["wo"][i][j] * att[j] for j in range(nq * hd)) for i in range(H)]
    hn = norm(h, w["ffn_norm"])
    gt, up = mv(w["wgate"], hn), mv(w["wup"], hn)
    a = [gt[j] / (1.0 + math.exp(-gt[j])) * up[j] for j in range(F)]
    return [h[i] + sum(w["wdown"][i][j] * a[j] for j in range(F)) for i in range(H)], k, v


@pytest.mark.parametrize("cfg", [TINY, TINY_QK], ids=["f32", "bf16-qknorm"])
def test_decode_step_matches_scalar_loops(cfg):
    run = RunConfig(batch=2, ctx0=(3, 5), steps=1, ctx_max=8, seed=7)
    raw = [gen.layer_weights(cfg, 7, l, gain_jitter=0.1) for l in range(cfg.n_layers)]
    glob = gen.global_weights(cfg, 7, gain_jitter=0.1)
    model = N.prepare(cfg, raw, glob)
    K, V = gen.kv_cache(cfg, run)
    toks = np.array([3, 9], dtype=np.int32)
    tr = N.decode_step(model, K.copy(), V.copy(), run.ctx0, tokens=toks)
    wl = [{k: N.to_f64(v).tolist() for k, v in r.items()} for r in raw]
    for b in range(2):
        x = N.to_f64(glob["embed"])[toks[b]].tolist()
        p = run.ctx0[b]
        for l in range(cfg.n_layers):
            Kc = [N.to_f64(K[l, b, g, :p]).tolist() for g in range(cfg.n_kv_heads)]
            Vc = [N.to_f64(V[l, b, g, :p]).tolist() for g in range(cfg.n_kv_heads)]
            x, _, _ = brute_layer(cfg, wl[l], x, Kc, Vc, p)
            if l + 1 < cfg.n_layers:
                assert N.max_rel_err(tr.x_in[l + 1][b], x) < 1e-12
        assert N.max_rel_err(tr.x_out[b], x) < 1e-12
        g = N.to_f64(glob["final_norm"])
        s = math.sqrt(sum(t * t for t in x) / len(x) + cfg.rms_eps)
        xn = [x[i] / s * g[i] for i in range(len(x))]
        lm = N.to_f64(glob["lm_head"])
        logits = [sum(lm[o][i] * xn[i] for i in range(len(x))) for o in range(cfg.vocab)]
        assert N.max_rel_err(tr.logits[b], logits) < 1e-12


def test_decode_writes_cache_at_position_in_storage_type():
    cfg = TINY_QK
    run = RunConfig(batch=1, ctx0=(4,), steps=1, ctx_max=8, seed=3)
    model = N.prepare(cfg, [gen.layer_weights(cfg, 3, 0)], gen.global_weights(cfg, 3))
    K, V = gen.kv_cache(cfg, run)
    K0 = K.copy()
    tr = N.decode_step(model, K, V, [4], tokens=np.array([2]))
    assert np.array_equal(K[0, 0, :, :4], K0[0, 0, :, :4])            # history untouched
    assert np.array_equal(K[0, 0, :, 5:], K0[0, 0, :, 5:])
    assert np.array_equal(K[0, 0, :, 4], N.store_like(tr.k[0][0], np.uint16))
    assert K.dtype == np.uint16


# ----------------------------------------------------------------------------- decode == prefill (P7)

@pytest.mark.parametrize("cfg", [TINY, TINY_QK], ids=["f32", "bf16-qknorm"])
def test_teacher_forced_decode_equals_causal_prefill(cfg):
    T = 7
    run = RunConfig(batch=1, ctx0=(0,), steps=T, ctx_max=T, seed=11, init_cache=False)
    model = N.prepare(cfg, [gen.layer_weights(cfg, 11, l, 0.1) for l in range(cfg.n_layers)],
                      gen.global_weights(cfg, 11, 0.1))
    toks = np.array([1, 5, 2, 2, 9, 0, 4], dtype=np.int32)
    Kp, Vp = gen.kv_cache(cfg, run)
    pre = N.prefill(model, Kp, Vp, toks)
    Kd, Vd = gen.kv_cache(cfg, run)
    for t in range(T):
        tr = N.decode_step(model, Kd, Vd, [t], tokens=toks[t:t + 1])
        for l in range(cfg.n_layers):
            assert N.max_rel_err(tr.x_in[l][0], pre.x_in[l][t]) < 1e-12
    assert N.max_rel_err(tr.logits[0], pre.logits[0]) < 1e-12
    assert np.array_equal(Kd, Kp) or N.max_rel_err(N.to_f64(Kd), N.to_f64(Kp)) < 1e-2


def test_argmax_lowest_index_wins_ties():
    a = np.array([[0.0, 3.0, 1.0, 3.0], [5.0, 5.0, 5.0, 5.0]])
    assert list(N.argmax_lowest(a)) == [1, 0]


# ----------------------------------------------------------------------------- error metric (R13)

def test_max_rel_err_hand_worked_values():
    # |diff| = (0, 0, 1), max |ref| = 4
    assert N.max_rel_err(np.array([1.0, 2.0, 3.0]), np.array([1.0, 2.0, 4.0])) == 0.25
    # an error in the negative direction counts as much as a positive one
    assert N.max_rel_err(np.array([0.5, 2.0]), np.array([1.0, 2.0])) == 0.25
    assert N.max_rel_err(np.array([1.0, 2.0]), np.array([0.5, 2.0])) == 0.25
    # the scale is the largest magnitude of the reference, negative entries included
    assert N.max_rel_err(np.array([-3.0, 1.0]), np.array([-4.0, 1.0])) == 0.25
    # the scale is the reference's, not the result's
    assert N.max_rel_err(np.array([8.0, 0.0]), np.array([4.0, 0.0])) == 1.0
    # an all-zero reference gives the absolute error
    assert N.max_rel_err(np.array([0.0, -1e-3]), np.array([0.0, 0.0])) == 1e-3
    # identical tensors, and empty ones
    assert N.max_rel_err(np.array([[1.5, -2.0]]), np.array([[1.5, -2.0]])) == 0.0
    assert N.max_rel_err(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0
    # a 2-D tensor is judged as a whole: max |diff| 0.5 over max |ref| 100
    got = np.array([[100.0, 0.0], [1.5, 0.0]])
    ref = np.array([[100.0, 0.0], [1.0, 0.0]])
    assert N.max_rel_err(got, ref) == 0.005
    with pytest.raises(ValueError):
        N.max_rel_err(np.zeros(3), np.zeros(4))


def test_max_rel_err_rows_judges_each_row_on_its_own_scale():
    got = np.array([[100.0, 0.0], [1.5, 0.0]])
    ref = np.array([[100.0, 0.0], [1.0, 0.0]])
    # row 0 is exact, row 1 is off by 0.5 against a scale of 1
    assert N.max_rel_err_rows(got, ref) == 0.5
    # rows of a 3-D tensor: row 1 has |diff| 2 over max |ref| 8
    ref3 = np.arange(16, dtype=np.float64).reshape(2, 2, 4) - 8.0
    got3 = ref3.copy()
    got3[1, 0, 0] -= 2.0
    assert N.max_rel_err_rows(got3, ref3) == 2.0 / 7.0
    got3[0, 1, 3] += 4.0
    assert N.max_rel_err_rows(got3, ref3) == 0.5
    assert N.max_rel_err_rows(np.zeros((0, 2)), np.zeros((0, 2))) == 0.0


@pytest.mark.parametrize("nq,nkv,S,hd", [(4, 2, 9, 8), (8, 8, 5, 4), (6, 1, 17, 6)])
def test_causal_attention_equals_one_position_at_a_time(nq, nkv, S, hd):
    """The masked score-matrix form of prefill attention against the decode
    attention of each position over its visible keys 0..i."""
    g = rng(nq * S)
    q = g.standard_normal((S, nq, hd))
    K = g.standard_normal((nkv, S, hd))
    V = g.standard_normal((nkv, S, hd))
    got = N.causal_attention(q, K, V)
    for i in range(S):
        want = N.attention(q[i], K[:, : i + 1], V[:, : i + 1])
        assert np.max(np.abs(got[i] - want)) < 1e-12
    # position 0 sees only key 0: the output is its value
    for h in range(nq):
        assert np.allclose(got[0, h], V[h // (nq // nkv), 0], atol=1e-15)


def test_float32_widening_runs_the_same_functions():
    """The CPU baseline's float32 model: weights widened exactly (bf16 values are
    fp32 values), and a step within fp32 rounding of the float64 oracle."""
    cfg = ModelConfig("t", 2, 64, 4, 2, 16, 96, 50, 1e-5, 1e4)
    run = RunConfig(batch=2, ctx0=(5, 9), steps=1, ctx_max=12, seed=3)
    raw = gen.all_layer_weights(cfg, 3, gain_jitter=0.1)
    glob = gen.global_weights(cfg, 3, gain_jitter=0.1)
    m64 = N.prepare(cfg, raw, glob)
    m32 = N.prepare(cfg, raw, glob, dtype=np.float32)
    assert m32.layers[0].wqkv.dtype == np.float32
    assert np.array_equal(m32.layers[1].wdown.astype(np.float64), m64.layers[1].wdown)
    K, V = gen.kv_cache(cfg, run)
    toks = gen.decode_tokens(cfg, run)[0]
    t64 = N.decode_step(m64, K.copy(), V.copy(), run.ctx0, tokens=toks)
    t32 = N.decode_step(m32, K.copy(), V.copy(), run.ctx0, tokens=toks)
    assert t32.logits.dtype == np.float32
    assert N.max_rel_err_rows(t32.logits, t64.logits) < 1e-5
