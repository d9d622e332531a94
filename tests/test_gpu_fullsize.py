"""GPU parity at the full workload shapes, end to end against the float64 oracle.

Each test runs whole steps of one workload on the GPU, in the launch
configuration the benchmark times (the workload's tile plan; one sub-queue per
worker for decode, shared sub-queues for prefill), and keeps a host copy of
every layer's intermediates after each step.  The oracle then streams the same
seeded model one layer at a time: each layer's weights are widened from their
seeded storage arrays and its cache rows regenerated from their seeds, and the
oracle's own hidden rows carry on to the next layer.  Nothing the GPU computed
feeds the oracle, so error that builds up over the layers shows.

Compared per layer and step: the attention output, the post-attention residual
rows (HRES), both branch outputs, the SwiGLU activation and the output rows
X_{l+1}; then the new cache entries, the final logits over the whole vocabulary
and the argmax of the GPU's logits.  Tolerance 2e-2 for these bf16 models, as
max |gpu - oracle| / max |oracle| per tensor, step and sequence: per row in
decode (each row is a sequence), per tensor in prefill (the rows are the
positions of one sequence).

The oracle's pass over the 36-layer, 2048-token prefill takes minutes, so it is
split over three tests of 12 layers that share one module state.
"""
import dataclasses
import gc
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import tile_synchronized_decoder_amd as T
from tile_synchronized_decoder_amd import device as D
import workloads as W
from oracle import numerics as N

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TOL = 2e-2
THREADS = 16
VOCAB_CHUNK = 16384


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _log(*a):
    from _gpucase import log
    log(*a)


_POOL = ThreadPoolExecutor(THREADS)


def widen_layer(raw):
    """The oracle's float64 layer, its tensors widened in parallel."""
    keys = list(raw)
    return N.Layer(**dict(zip(keys, _POOL.map(N.widen, [raw[k] for k in keys]))))


def oracle_logits(m, raw_global, x):
    """N.lm_head over the vocabulary in chunks of rows (same values, bounded memory)."""
    g = N.widen(raw_global["final_norm"])
    W_lm = raw_global["lm_head"]
    out = np.empty((x.shape[0], m.vocab))
    for v0 in range(0, m.vocab, VOCAB_CHUNK):
        out[:, v0:v0 + VOCAB_CHUNK] = N.lm_head(m, x, g, N.widen(W_lm[v0:v0 + VOCAB_CHUNK]))
    return out


class Snap:
    """Host copy of a workspace after one step: every layer's fp32 tensors."""

    def __init__(self, ws: torch.Tensor, q: T.Queue, rows: int):
        self.host = ws.cpu()
        self.q, self.rows = q, rows

    def get(self, kind, layer, cols):
        off = self.q.workspace_offset(kind, layer)
        n = self.rows * cols
        return self.host[off: off + 4 * n].view(torch.float32).numpy().reshape(self.rows, cols).astype(np.float64)


def compare_layer(errs, tag, snap: Snap, m, l, lt: N.LayerTrace, per_row=True):
    """Decode: each row is a sequence, judged on its own scale.  Prefill: the
    rows are the positions of one sequence, so each tensor is judged whole
    (max |gpu - oracle| / max |oracle| per tensor, per step, per sequence)."""
    rel = N.max_rel_err_rows if per_row else N.max_rel_err
    x_in, h = snap.get(T.MK_T_X, l, m.hidden), snap.get(T.MK_T_HRES, l, m.hidden)
    x_out = snap.get(T.MK_T_X, l + 1, m.hidden)
    errs[f"{tag}att{l}"] = rel(snap.get(T.MK_T_ATT, l, m.attn_cols), lt.attn)
    errs[f"{tag}h{l}"] = rel(h, lt.h)
    errs[f"{tag}attn_branch{l}"] = rel(h - x_in, lt.attn_branch)
    errs[f"{tag}act{l}"] = rel(snap.get(T.MK_T_ACT, l, m.ffn), lt.act)
    errs[f"{tag}mlp_branch{l}"] = rel(x_out - h, lt.mlp_branch)
    errs[f"{tag}x{l + 1}"] = rel(x_out, lt.x_out)


def check(errs, what):
    worst = max(errs, key=errs.get)
    _log(f"    {what}: worst {worst} = {errs[worst]:.3e}")
    assert errs[worst] <= TOL, {k: v for k, v in errs.items() if v > TOL}


_CACHE = {}


def _weights(m, seed):
    """Seeded host weights (storage arrays) and their device copy, one model at a time."""
    key = (m.name, seed)
    if key not in _CACHE:
        _CACHE.clear()
        gc.collect()
        torch.cuda.empty_cache()
        raw_layers = W.gen.all_layer_weights(m, seed, threads=THREADS)
        raw_global = W.gen.global_weights(m, seed)
        _CACHE[key] = (raw_layers, raw_global, D.upload_weights(raw_layers, raw_global))
    return _CACHE[key]


class Decoder:
    """Device state of one decode workload at its full shape."""

    def __init__(self, wl: W.Workload, dm, dkv=None, ctx0=None):
        m, r = wl.model, wl.run
        self.wl, self.m, self.r, self.dm = wl, m, r, dm
        self.ctx0 = list(ctx0 if ctx0 is not None else r.ctx0)
        if dkv is None:
            K, V = W.gen.kv_cache(m, r, threads=THREADS)
            dkv = D.upload_kv(K, V)
            del K, V
        self.dkv = dkv
        self.tokens = W.gen.decode_tokens(m, r)
        self.q = T.mk_build_queue(T.make_config(m), T.make_plan(wl.plan, T.MK_DECODE, r.batch, r.ctx_max))
        self.dq = D.upload_queue(self.q)
        self.ws = D.workspace(self.q)
        self.logits = torch.zeros((r.batch, m.vocab), dtype=torch.float32, device="cuda")
        self.nxt = torch.zeros((r.batch,), dtype=torch.int32, device="cuda")

    def ctx(self, t):
        return [p + t for p in self.ctx0]

    def step(self, t, mode=T.MK_MEGAKERNEL):
        """Decode step t; returns the host snapshot, logits and argmax."""
        T.mk_decode_step(self.q, self.dq, self.dm.w, self.dkv.kv,
                         torch.from_numpy(self.tokens[t].astype(np.int32)).cuda(), None,
                         torch.tensor(self.ctx(t), dtype=torch.int32, device="cuda"), self.r.batch, self.ws,
                         self.logits, self.nxt, mode)
        torch.cuda.synchronize()
        e = T.mk_device_error(self.q, self.ws)
        assert e.code == 0, (e.code, e.instr, e.barrier, e.value, e.target)
        lg = self.logits.cpu().numpy().astype(np.float64)
        nx = self.nxt.cpu().numpy()
        assert np.array_equal(nx, N.argmax_lowest(self.logits.cpu().numpy())), "argmax of the GPU logits"
        return Snap(self.ws, self.q, self.r.batch), lg

    def new_cache_entries(self, steps):
        """GPU cache rows written by steps 0..steps-1: [steps][L, B, nkv, hd] bf16 bits, K and V."""
        out = []
        for t in range(steps):
            ks, vs = [], []
            for b, p in enumerate(self.ctx(t)):
                ks.append(self.dkv.k[:, b, :, p].cpu().numpy().view(np.uint16))
                vs.append(self.dkv.v[:, b, :, p].cpu().numpy().view(np.uint16))
            out.append((np.stack(ks, 1), np.stack(vs, 1)))
        return out


def stream_decode(d: Decoder, raw_layers, raw_global, snaps, logits, kv_new, tag=""):
    """The oracle over steps 0..len(snaps)-1 of a decode workload, one layer at a time."""
    m, r = d.m, d.r
    steps = len(snaps)
    embed = raw_global["embed"]
    xs = [N.widen(embed[d.tokens[t]]) for t in range(steps)]
    for l in range(m.n_layers):
        errs = {}
        lw = widen_layer(raw_layers[l])
        K, V = W.gen.kv_cache_layer(m, r, l, threads=THREADS)
        for t in range(steps):
            ctx = d.ctx(t)
            lt = N.decode_layer(m, lw, xs[t], K, V, ctx)
            compare_layer(errs, f"{tag}s{t}.", snaps[t], m, l, lt)
            xs[t] = lt.x_out
            for b, p in enumerate(ctx):
                errs[f"{tag}s{t}.k{l}"] = max(errs.get(f"{tag}s{t}.k{l}", 0.0),
                                             N.max_rel_err(N.widen(kv_new[t][0][l, b]), N.widen(K[b, :, p])))
                errs[f"{tag}s{t}.v{l}"] = max(errs.get(f"{tag}s{t}.v{l}", 0.0),
                                             N.max_rel_err(N.widen(kv_new[t][1][l, b]), N.widen(V[b, :, p])))
        check(errs, f"{d.wl.name} layer {l}")
        del lw, K, V
    errs = {}
    for t in range(steps):
        errs[f"{tag}s{t}.x_out"] = N.max_rel_err_rows(snaps[t].get(T.MK_T_X, m.n_layers, m.hidden), xs[t])
        errs[f"{tag}s{t}.logits"] = N.max_rel_err_rows(logits[t], oracle_logits(m, raw_global, xs[t]))
    check(errs, f"{d.wl.name} logits")


@pytest.mark.parametrize("name,steps", [("llama8b_b1", 2), ("llama8b_b4", 1), ("llama8b_b16", 1)])
def test_llama8b_decode_end_to_end(name, steps):
    """Llama-3-8B shape at context 4096, batch 1 / 4 / 16, all 32 layers and the
    LM head; at batch 4 the kernel-per-op step is also bit-identical to the
    megakernel's."""
    wl = W.WORKLOADS[name]
    _log(f"[fullsize] {name}: {steps} step(s), plan {wl.plan}")
    raw_layers, raw_global, dm = _weights(wl.model, wl.run.seed)
    d = Decoder(wl, dm)
    snaps, logits = zip(*[d.step(t) for t in range(steps)])
    kv_new = d.new_cache_entries(steps)
    if wl.run.batch == 4:
        # restore the cache, then the same step once per op
        K, V = W.gen.kv_cache(wl.model, wl.run, threads=THREADS)
        d.dkv.k.copy_(torch.from_numpy(K.view(np.int16)))
        d.dkv.v.copy_(torch.from_numpy(V.view(np.int16)))
        del K, V
        s_kpo, lg_kpo = d.step(0, T.MK_KERNEL_PER_OP)
        assert np.array_equal(lg_kpo, logits[0])
        assert torch.equal(s_kpo.host, snaps[0].host)
    del d.dkv
    torch.cuda.empty_cache()
    stream_decode(d, raw_layers, raw_global, list(snaps), list(logits), kv_new)


def test_llama1b_stream_b32_end_to_end():
    """Batch 32 with per-sequence contexts U{256..8192}: two consecutive steps,
    all 16 layers and the LM head."""
    wl = W.WORKLOADS["llama1b_stream_b32"]
    _log(f"[fullsize] {wl.name} contexts {min(wl.run.ctx0)}..{max(wl.run.ctx0)}")
    raw_layers, raw_global, dm = _weights(wl.model, wl.run.seed)
    d = Decoder(wl, dm)
    snaps, logits = zip(*[d.step(t) for t in range(2)])
    kv_new = d.new_cache_entries(2)
    del d.dkv
    torch.cuda.empty_cache()
    stream_decode(d, raw_layers, raw_global, list(snaps), list(logits), kv_new)


# ----------------------------------------------------------------------------- Qwen3-8B: prefill, then decode

class QwenRun:
    """GPU prefill of 2048 tokens and two decode steps on the cache it wrote,
    then the oracle's matching pass, advanced a chunk of layers per test."""

    DECODE_STEPS = 2

    def __init__(self):
        wl = W.WORKLOADS["qwen8b_prefill"]
        m, r = wl.model, wl.run
        self.wl, self.m, self.r, self.S = wl, m, r, r.prefill_len
        self.raw_layers, self.raw_global, dm = _weights(m, r.seed)
        S = self.S
        K, V = W.gen.kv_cache(m, r)                   # empty cache, one row
        dkv = D.upload_kv(K, V)
        del K, V
        self.ptok = W.gen.prefill_tokens(m, r)
        qp = T.mk_build_queue(T.make_config(m), T.make_plan(wl.plan.for_prefill(), T.MK_PREFILL, S, r.ctx_max))
        dqp, wsp = D.upload_queue(qp), D.workspace(qp)
        plg = torch.zeros((m.vocab,), dtype=torch.float32, device="cuda")
        pnx = torch.zeros((1,), dtype=torch.int32, device="cuda")
        T.mk_prefill(qp, dqp, dm.w, dkv.kv, torch.from_numpy(self.ptok).cuda(), S, 0, wsp, plg, pnx,
                     T.MK_MEGAKERNEL)
        torch.cuda.synchronize()
        e = T.mk_device_error(qp, wsp)
        assert e.code == 0, (e.code, e.instr, e.barrier)
        self.psnap = Snap(wsp, qp, S)
        self.plogits = plg.cpu().numpy()[None, :].astype(np.float64)
        assert int(pnx.item()) == int(N.argmax_lowest(plg.cpu().numpy()[None, :])[0])
        del wsp
        torch.cuda.empty_cache()
        _log("    prefill done on the GPU")
        wl_dec = dataclasses.replace(wl, run=dataclasses.replace(r, ctx0=(S,)))
        self.dec = Decoder(wl_dec, dm, dkv=dkv, ctx0=[S])
        self.dsnaps, self.dlogits = map(list, zip(*[self.dec.step(t) for t in range(self.DECODE_STEPS)]))
        self.Kg = dkv.k.cpu().numpy().view(np.uint16)             # [L, 1, nkv, ctx_max, hd]
        self.Vg = dkv.v.cpu().numpy().view(np.uint16)
        del self.dec.dkv, dkv
        torch.cuda.empty_cache()
        # oracle state: the prefill rows and each decode step's row, at the next layer
        self.next_layer = 0
        self.xp = N.widen(self.raw_global["embed"][self.ptok])
        self.xd = [N.widen(self.raw_global["embed"][self.dec.tokens[t]]) for t in range(self.DECODE_STEPS)]

    def advance(self, layers):
        """Stream the oracle over `layers`; every layer is compared and logged
        before the chunk's verdict, so one run shows the whole error profile."""
        m, S = self.m, self.S
        assert layers[0] == self.next_layer, "the chunks run in order"
        over = {}
        for l in layers:
            errs = {}
            lw = widen_layer(self.raw_layers[l])
            K = np.zeros((1, m.n_kv_heads, self.r.ctx_max, m.head_dim), dtype=np.uint16)
            V = np.zeros_like(K)
            lt = N.prefill_layer(m, lw, self.xp, K, V, row=0)
            compare_layer(errs, "prefill.", self.psnap, m, l, lt, per_row=False)
            # per position, for information (stricter than the per-sequence reading)
            pos = {k: N.max_rel_err_rows(self.psnap.get(kind, l1, cols), ref) for k, kind, l1, cols, ref in (
                ("att", T.MK_T_ATT, l, m.attn_cols, lt.attn), ("act", T.MK_T_ACT, l, m.ffn, lt.act),
                ("x", T.MK_T_X, l + 1, m.hidden, lt.x_out))}
            self.xp = lt.x_out
            for t in range(self.DECODE_STEPS):
                lt = N.decode_layer(m, lw, self.xd[t], K, V, [S + t])
                compare_layer(errs, f"s{t}.", self.dsnaps[t], m, l, lt)
                self.xd[t] = lt.x_out
            n = S + self.DECODE_STEPS
            errs[f"k{l}"] = N.max_rel_err(N.widen(self.Kg[l, 0, :, :n]), N.widen(K[0, :, :n]))
            errs[f"v{l}"] = N.max_rel_err(N.widen(self.Vg[l, 0, :, :n]), N.widen(V[0, :, :n]))
            self.next_layer = l + 1
            worst = max(errs, key=errs.get)
            _log(f"    qwen8b layer {l}: worst {worst} = {errs[worst]:.3e}; x{l + 1} {errs[f'prefill.x{l + 1}']:.3e}; "
                 f"per position: " + ", ".join(f"{k} {v:.2e}" for k, v in pos.items()))
            over.update({k: v for k, v in errs.items() if v > TOL})
        assert not over, over

    def finish(self):
        m = self.m
        assert self.next_layer == m.n_layers
        errs = {"prefill.x_out": N.max_rel_err(self.psnap.get(T.MK_T_X, m.n_layers, m.hidden), self.xp),
                "prefill.logits": N.max_rel_err_rows(self.plogits, oracle_logits(m, self.raw_global, self.xp[-1:]))}
        for t in range(self.DECODE_STEPS):
            errs[f"s{t}.x_out"] = N.max_rel_err_rows(self.dsnaps[t].get(T.MK_T_X, m.n_layers, m.hidden), self.xd[t])
            errs[f"s{t}.logits"] = N.max_rel_err_rows(self.dlogits[t], oracle_logits(m, self.raw_global, self.xd[t]))
        check(errs, "qwen8b logits")


@pytest.fixture(scope="module")
def qwen():
    _log("[fullsize] qwen8b_prefill: prefill 2048 then 2 decode steps")
    return QwenRun()


@pytest.mark.parametrize("chunk", [0, 1, 2])
def test_qwen8b_prefill_then_decode_end_to_end(qwen, chunk):
    """Qwen3-8B shape with QK-norm: the 2048-token prefill (every position of
    every layer, and the cache it writes) and two decode steps after it; layers
    12 * chunk .. 12 * chunk + 11, then the logits with the last chunk."""
    qwen.advance(list(range(12 * chunk, 12 * chunk + 12)))
    if chunk == 2:
        qwen.finish()
