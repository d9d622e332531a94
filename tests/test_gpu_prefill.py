"""GPU parity of the prefill path (matrix-core GEMM tiles and causal attention
tiles) through the C ABI against the float64 oracle.

The GEMM tiles round activations to bf16 on their way into the matrix cores
and accumulate in fp32; the attention tile rounds Q and the probabilities to
bf16.  Tolerance: max |gpu - oracle| / max |oracle| <= 2e-2 per tensor, as for
the bf16 decode path.  Megakernel and kernel-per-op runs execute the same tile
bodies and must agree bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import tile_synchronized_decoder_amd as T
from tile_synchronized_decoder_amd import device as D
import workloads as W
from oracle import numerics as N

pytestmark = pytest.mark.gpu

TOL = 2e-2

# A Qwen3-shaped model narrowed to two layers so the oracle finishes in seconds:
# head_dim 128, GQA 4/2, per-head QK RMSNorm, rope theta 1e6.
SMALL = W.ModelConfig(name="qwen-shaped-small", n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=2,
                      head_dim=128, ffn=768, vocab=1000, rms_eps=1e-6, rope_theta=1e6, qk_norm=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from _gpucase import log
    log(f"[gpu] {torch.cuda.get_device_name(0)} lib={T.library_path()}")


class PrefillCase:
    """Weights, an empty cache of `kv_rows` sequences and a prefill queue for S_max rows."""

    def __init__(self, m: W.ModelConfig, s_max: int, ctx_max: int, kv_rows: int, seed: int, jitter=0.1):
        from _gpucase import log
        self.m, self.s_max, self.ctx_max, self.kv_rows = m, s_max, ctx_max, kv_rows
        log(f"[prefill case] {m.name}: L={m.n_layers} H={m.hidden} S_max={s_max} ctx_max={ctx_max} "
            f"kv_rows={kv_rows} seed={seed}")
        self.run = W.RunConfig(batch=kv_rows, ctx0=(0,) * kv_rows, steps=4, ctx_max=ctx_max, seed=seed,
                               prefill_len=s_max, init_cache=False)
        self.raw_layers = W.gen.all_layer_weights(m, seed, jitter)
        self.raw_global = W.gen.global_weights(m, seed, jitter)
        self.K0, self.V0 = W.gen.kv_cache(m, self.run)
        self.tokens = W.gen.prefill_tokens(m, self.run)
        self.q = T.mk_build_queue(T.make_config(m), T.make_plan(W.Plan(), T.MK_PREFILL, s_max, ctx_max))
        self.dq = D.upload_queue(self.q)
        self.dm = D.upload_weights(self.raw_layers, self.raw_global)
        self.dkv = D.upload_kv(self.K0, self.V0)
        self.ws = D.workspace(self.q)
        self.logits = torch.zeros((m.vocab,), dtype=torch.float32, device="cuda")
        self.nxt = torch.zeros((1,), dtype=torch.int32, device="cuda")
        self.model = N.prepare(m, self.raw_layers, self.raw_global)

    def reset(self):
        self.dkv.k.copy_(torch.from_numpy(self.K0.view(np.int16)))
        self.dkv.v.copy_(torch.from_numpy(self.V0.view(np.int16)))
        self.ws.zero_()
        self.logits.zero_()
        self.nxt.zero_()

    def prefill(self, seq_len: int, kv_row: int, mode: int, tokens=None):
        tok = self.tokens[:seq_len] if tokens is None else tokens
        dt = torch.from_numpy(np.ascontiguousarray(tok, dtype=np.int32)).cuda()
        T.mk_prefill(self.q, self.dq, self.dm.w, self.dkv.kv, dt, seq_len, kv_row, self.ws, self.logits,
                     self.nxt, mode)
        torch.cuda.synchronize()
        e = T.mk_device_error(self.q, self.ws)
        assert e.code == 0, (e.code, e.instr, e.barrier, e.value, e.target)

    def tensor(self, kind: int, layer: int, cols: int, rows: int) -> np.ndarray:
        return D.ws_view(self.ws, self.q, kind, layer, (self.s_max, cols))[:rows].cpu().numpy().astype(np.float64)

    def snapshot(self, seq_len: int) -> dict:
        m = self.m
        out = {}
        for l in range(m.n_layers + 1):
            out[f"x{l}"] = self.tensor(T.MK_T_X, l, m.hidden, seq_len)
        for l in range(m.n_layers):
            out[f"qkv{l}"] = self.tensor(T.MK_T_QKV, l, m.qkv_cols, seq_len)
            out[f"att{l}"] = self.tensor(T.MK_T_ATT, l, m.attn_cols, seq_len)
            out[f"h{l}"] = self.tensor(T.MK_T_HRES, l, m.hidden, seq_len)
            out[f"act{l}"] = self.tensor(T.MK_T_ACT, l, m.ffn, seq_len)
        k, v = D.kv_to_host(self.dkv, np.uint16)
        out["k"], out["v"] = k.copy(), v.copy()
        out["logits"] = self.logits.cpu().numpy().astype(np.float64)
        out["next"] = self.nxt.cpu().numpy().copy()
        return out


def oracle_prefill(c: PrefillCase, seq_len: int, kv_row: int, tokens=None):
    K, V = c.K0.copy(), c.V0.copy()
    tok = c.tokens[:seq_len] if tokens is None else tokens
    tr = N.prefill(c.model, K, V, tok, row=kv_row)
    return tr, K, V


def compare(c: PrefillCase, got: dict, tr, Kref, Vref, seq_len: int, kv_row: int):
    from _gpucase import log
    m = c.m
    nq, nkv, hd = m.n_q_heads, m.n_kv_heads, m.head_dim
    errs = {}
    for l in range(m.n_layers):
        errs[f"x_in{l}"] = N.max_rel_err(got[f"x{l}"], tr.x_in[l])
        q = got[f"qkv{l}"][:, : nq * hd].reshape(seq_len, nq, hd)
        errs[f"q{l}"] = N.max_rel_err(q, tr.q[l])
        errs[f"att{l}"] = N.max_rel_err(got[f"att{l}"], tr.attn[l])
        errs[f"h{l}"] = N.max_rel_err(got[f"h{l}"], tr.h[l])
        errs[f"attn_branch{l}"] = N.max_rel_err(got[f"h{l}"] - got[f"x{l}"], tr.attn_branch[l])
        errs[f"act{l}"] = N.max_rel_err(got[f"act{l}"], tr.act[l])
        errs[f"mlp_branch{l}"] = N.max_rel_err(got[f"x{l + 1}"] - got[f"h{l}"], tr.mlp_branch[l])
        gk = N.bf16_bits_to_f64(got["k"][l, kv_row, :, :seq_len])
        gv = N.bf16_bits_to_f64(got["v"][l, kv_row, :, :seq_len])
        errs[f"kcache{l}"] = N.max_rel_err(gk, N.bf16_bits_to_f64(Kref[l, kv_row, :, :seq_len]))
        errs[f"vcache{l}"] = N.max_rel_err(gv, N.bf16_bits_to_f64(Vref[l, kv_row, :, :seq_len]))
    errs["x_out"] = N.max_rel_err(got[f"x{m.n_layers}"], tr.x_out)
    errs["logits"] = N.max_rel_err(got["logits"][None, :], tr.logits)
    worst = max(errs, key=errs.get)
    log(f"    S={seq_len} row={kv_row}: worst {worst} = {errs[worst]:.3e}")
    assert errs[worst] <= TOL, errs
    # the argmax follows the GPU's own logits (lowest index on ties)
    assert int(got["next"][0]) == int(N.argmax_lowest(got["logits"].astype(np.float32)[None, :])[0])
    # cache entries outside [0, seq_len) of row kv_row, and the other rows, are untouched
    mask = np.ones(got["k"].shape, dtype=bool)
    mask[:, kv_row, :, :seq_len] = False
    assert not got["k"][mask].any() and not got["v"][mask].any(), "prefill wrote outside its cache slots"


@pytest.fixture(scope="module")
def small():
    return PrefillCase(SMALL, s_max=256, ctx_max=320, kv_rows=2, seed=11)


@pytest.mark.parametrize("seq_len,kv_row", [(200, 1), (256, 0), (1, 1), (129, 0)])
def test_prefill_parity_both_modes(small, seq_len, kv_row):
    """Ragged tails (200, 129), full blocks (256) and a single token, each in
    both execution modes; the two modes agree bit for bit."""
    tr, K, V = oracle_prefill(small, seq_len, kv_row)
    snaps = {}
    for mode, name in ((T.MK_MEGAKERNEL, "mega"), (T.MK_KERNEL_PER_OP, "kpo")):
        small.reset()
        small.prefill(seq_len, kv_row, mode)
        snaps[name] = small.snapshot(seq_len)
        compare(small, snaps[name], tr, K, V, seq_len, kv_row)
    for key in snaps["mega"]:
        assert np.array_equal(snaps["mega"][key], snaps["kpo"][key]), f"modes differ in {key}"


def test_prefill_repeat_is_deterministic(small):
    """Two megakernel runs on the same inputs give identical bits (the work
    queue's order of execution varies, the arithmetic of each tile does not)."""
    out = []
    for _ in range(2):
        small.reset()
        small.prefill(200, 1, T.MK_MEGAKERNEL)
        out.append(small.snapshot(200))
    for key in out[0]:
        assert np.array_equal(out[0][key], out[1][key]), key


def test_prefill_then_decode(small):
    """Prefill 200 tokens, then three decode steps on the cache it wrote; the
    decode logits follow the oracle's own prefill-then-decode chain."""
    from _gpucase import log
    m, S = SMALL, 200
    small.reset()
    small.prefill(S, 0, T.MK_MEGAKERNEL)
    # oracle chain on a cache with one row
    K = np.zeros((m.n_layers, 1, m.n_kv_heads, small.ctx_max, m.head_dim), dtype=np.uint16)
    V = np.zeros_like(K)
    N.prefill(small.model, K, V, small.tokens[:S], row=0)
    # the GPU cache row 0 becomes a one-row decode cache
    dk = small.dkv.k[:, :1].contiguous()
    dv = small.dkv.v[:, :1].contiguous()
    kv = T.mk_kv()
    kv.k, kv.v, kv.rows = dk.data_ptr(), dv.data_ptr(), 1
    qd = T.mk_build_queue(T.make_config(m), T.make_plan(W.Plan(), T.MK_DECODE, 1, small.ctx_max))
    dqd = D.upload_queue(qd)
    wsd = D.workspace(qd)
    logits = torch.zeros((1, m.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.zeros((1,), dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(12)
    for t in range(3):
        tok = rng.integers(0, m.vocab, size=(1,)).astype(np.int32)
        tr = N.decode_step(small.model, K, V, [S + t], tokens=tok)
        T.mk_decode_step(qd, dqd, small.dm.w, kv, torch.from_numpy(tok).cuda(), None,
                         torch.tensor([S + t], dtype=torch.int32, device="cuda"), 1, wsd, logits, nxt,
                         T.MK_MEGAKERNEL)
        torch.cuda.synchronize()
        err = N.max_rel_err(logits.cpu().numpy().astype(np.float64), tr.logits)
        log(f"    decode step {t} after prefill: logits err {err:.3e}")
        assert err <= TOL


def test_prefill_rejects_bad_calls(small):
    small.reset()
    tok = torch.zeros((small.s_max + 1,), dtype=torch.int32, device="cuda")
    with pytest.raises(T.MkError):        # longer than the queue's S_max
        T.mk_prefill(small.q, small.dq, small.dm.w, small.dkv.kv, tok, small.s_max + 1, 0, small.ws,
                     small.logits, small.nxt, T.MK_MEGAKERNEL)
    with pytest.raises(T.MkError):        # cache row outside the cache
        T.mk_prefill(small.q, small.dq, small.dm.w, small.dkv.kv, tok, 10, small.kv_rows, small.ws,
                     small.logits, small.nxt, T.MK_MEGAKERNEL)
    with pytest.raises(T.MkError):        # workspace too small
        T.mk_prefill(small.q, small.dq, small.dm.w, small.dkv.kv, tok, 10, 0, small.ws[:1024],
                     small.logits, small.nxt, T.MK_MEGAKERNEL)


def test_prefill_bad_token_reports_device_error(small):
    """A token id outside the vocabulary is caught by the embedding tile, which
    records the error; the run still completes."""
    small.reset()
    tok = small.tokens[:64].copy()
    tok[5] = SMALL.vocab + 3
    dt = torch.from_numpy(tok.astype(np.int32)).cuda()
    T.mk_prefill(small.q, small.dq, small.dm.w, small.dkv.kv, dt, 64, 0, small.ws, small.logits, small.nxt,
                 T.MK_MEGAKERNEL)
    e = T.mk_device_error(small.q, small.ws)
    assert e.code == 4 and e.barrier == 5 and e.value == SMALL.vocab + 3


def test_prefill_rejects_hidden_not_multiple_of_128(small):
    """The embedding and GEMM epilogues sum squares over 128-column groups of the
    hidden rows: a hidden size of 192 is refused before anything runs."""
    m = dataclasses.replace(SMALL, name="qwen-shaped-h192", hidden=192)
    plan = W.Plan(bm=128, bn=128)
    q = T.mk_build_queue(T.make_config(m), T.make_plan(plan, T.MK_PREFILL, 128, 256))
    tok = torch.zeros((128,), dtype=torch.int32, device="cuda")
    with pytest.raises(T.MkError) as ei:
        T.mk_prefill(q, small.dq, small.dm.w, small.dkv.kv, tok, 16, 0, small.ws, small.logits, small.nxt,
                     T.MK_MEGAKERNEL)
    assert ei.value.status == T.MK_ENOTSUP


@pytest.mark.parametrize("lo_mask", [0, 7, 11])
def test_prefill_hi_parts_only_meets_oracle(small, lo_mask):
    """GEMMs whose bit is clear in MK_OPT_PREFILL_LO take the hi parts of their
    activations only (rounded to bf16): the result changes against taking both
    parts, still meets the oracle on the short model in both modes, and the two
    modes agree bit for bit."""
    seq_len, kv_row = 200, 1
    tr, K, V = oracle_prefill(small, seq_len, kv_row)
    small.reset()
    small.prefill(seq_len, kv_row, T.MK_MEGAKERNEL)
    both = small.snapshot(seq_len)
    snaps = {}
    T.mk_set_option(T.MK_OPT_PREFILL_LO, lo_mask)
    try:
        for mode, name in ((T.MK_MEGAKERNEL, "mega"), (T.MK_KERNEL_PER_OP, "kpo")):
            small.reset()
            small.prefill(seq_len, kv_row, mode)
            snaps[name] = small.snapshot(seq_len)
            compare(small, snaps[name], tr, K, V, seq_len, kv_row)
    finally:
        T.mk_set_option(T.MK_OPT_PREFILL_LO, 15)
    for key in snaps["mega"]:
        assert np.array_equal(snaps["mega"][key], snaps["kpo"][key]), f"modes differ in {key}"
    last = f"x{small.m.n_layers}"
    assert not np.array_equal(snaps["mega"][last], both[last]), "the option changed nothing"
