"""Multi-stream mode (MK_MULTI_STREAM) on the GPU.

One kernel per (layer, op) segment, dealt round-robin to several streams;
every instruction waits on and signals the megakernel's tile counters, so a
segment runs while the one before it still does.  The op bodies and the tile
schedule are the megakernel's, so every output (each layer's intermediates,
the new cache entries, logits, argmax) must equal the megakernel's bit for
bit, for 1 to 4 streams, with static and shared sub-queue plans and with fused
split combines; also with a NaN-poisoned workspace and seeded producer delays.
One multi-step case is also checked against the float64 oracle directly
(tolerance 2e-2 per row, bf16 model).
"""
import dataclasses

import numpy as np
import pytest
import torch

import tile_synchronized_decoder_amd as T
import workloads as W
from oracle import numerics as N

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(autouse=True)
def _restore_options():
    yield
    T.mk_set_option(T.MK_OPT_STREAMS, 2)
    T.mk_set_option(T.MK_OPT_DELAY_SEED, 0)


def _cases():
    ncu = 256
    f32 = W.WORKLOADS["layer256_f32"]
    base = W.shrink(W.WORKLOADS["llama1b_b1"], n_layers=2, vocab=4096, batch=1, ctx0=(1024,), steps=1)
    b4 = W.shrink(W.WORKLOADS["llama1b_b1"], n_layers=2, vocab=4096, batch=4, ctx0=(1024, 37, 600, 1),
                  steps=1, name="llama1b_L2_B4")
    return {
        "f32_layer": f32,
        "bf16_1b_b1_static": dataclasses.replace(base, plan=W.Plan(tf=32, td=8, n_queues=ncu)),
        "bf16_1b_b4_shared8": dataclasses.replace(b4, plan=W.Plan(n_queues=8)),
        "bf16_1b_b1_fused": dataclasses.replace(base, plan=W.Plan(tf=32, td=8, n_queues=ncu, fuse_combine=1)),
    }


def _outputs(c):
    m = c.m
    out = {f"x{l}": c.tensor(T.MK_T_X, l, m.hidden) for l in range(m.n_layers + 1)}
    for l in range(m.n_layers):
        out[f"qkv{l}"] = c.tensor(T.MK_T_QKV, l, m.qkv_cols)
        if not c.wl.plan.fuse_combine:
            out[f"att{l}"] = c.tensor(T.MK_T_ATT, l, m.attn_cols)
        out[f"h{l}"] = c.tensor(T.MK_T_HRES, l, m.hidden)
        out[f"act{l}"] = c.tensor(T.MK_T_ACT, l, m.ffn)
    if c.logits is not None:
        out["logits"] = c.logits.cpu().numpy().copy()
        out["next"] = c.nxt.cpu().numpy().copy()
    k, v = c.kv_host()
    out["k"], out["v"] = k.copy(), v.copy()
    return out


def _run(c, mode, poison=False, seed=0):
    c.reset_kv()
    if poison:
        c.ws.fill_(255)
        if c.logits is not None:
            c.logits.fill_(float("nan"))
            c.nxt.fill_(-1)
    T.mk_set_option(T.MK_OPT_DELAY_SEED, seed)
    try:
        c.step(0, list(c.wl.run.ctx0), mode)
    finally:
        T.mk_set_option(T.MK_OPT_DELAY_SEED, 0)
    err = T.mk_device_error(c.q, c.ws)
    assert err.code == 0, (err.code, err.instr, err.barrier, err.value, err.target)
    if mode != T.MK_KERNEL_PER_OP:
        tg = np.frombuffer(c.q.export(T.MK_PART_TARGETS), dtype=np.uint32)
        assert np.array_equal(c.counters(), tg), "counters must end at their targets"
    return _outputs(c)


def _diff(a, b):
    return [k for k in a if not np.array_equal(a[k], b[k])]


@pytest.mark.parametrize("name", list(_cases()))
def test_multi_stream_equals_megakernel_bitwise(name):
    from _gpucase import make_case, log
    c = make_case(_cases()[name], gain_jitter=0.1)
    ref = _run(c, T.MK_MEGAKERNEL)
    for k, v in ref.items():
        if v.dtype.kind == "f":
            assert np.isfinite(v).all(), k
    assert not _diff(ref, _run(c, T.MK_KERNEL_PER_OP))
    for streams in (1, 2, 3, 4):
        T.mk_set_option(T.MK_OPT_STREAMS, streams)
        bad = _diff(ref, _run(c, T.MK_MULTI_STREAM))
        log(f"    {name} streams={streams}: {'identical' if not bad else 'DIFFERS in ' + ','.join(bad[:6])}")
        assert not bad, (streams, bad)


@pytest.mark.parametrize("name", ["bf16_1b_b1_static", "bf16_1b_b4_shared8"])
def test_multi_stream_poisoned_and_delayed_runs_are_bit_identical(name):
    from _gpucase import make_case, log
    c = make_case(_cases()[name], gain_jitter=0.1)
    T.mk_set_option(T.MK_OPT_STREAMS, 3)
    clean = _run(c, T.MK_MULTI_STREAM)
    for seed in (1, 2):
        bad = _diff(clean, _run(c, T.MK_MULTI_STREAM, poison=True, seed=seed))
        log(f"    {name} seed {seed}: {'identical' if not bad else 'DIFFERS in ' + ','.join(bad[:6])}")
        assert not bad, (seed, bad)


def test_multi_stream_multistep_matches_oracle():
    """Three teacher-forced steps at batch 3 with ragged contexts (the caller
    advances the context lengths) against the float64 oracle."""
    from _gpucase import make_case, log
    wl = W.shrink(W.WORKLOADS["llama1b_b1"], n_layers=2, vocab=4096, batch=3, ctx0=(900, 31, 511), steps=3,
                  name="llama1b_L2_B3_ms")
    c = make_case(wl, gain_jitter=0.1)
    c.reset_kv()
    model = c.oracle_model()
    K, V = c.K0.copy(), c.V0.copy()
    worst = 0.0
    for t in range(3):
        ctx = [p + t for p in wl.run.ctx0]
        c.step(t, ctx, T.MK_MULTI_STREAM)
        tr = N.decode_step(model, K, V, ctx, tokens=c.tokens[t])
        worst = max(worst, N.max_rel_err_rows(c.logits.cpu().numpy().astype(np.float64), tr.logits),
                    N.max_rel_err_rows(c.tensor(T.MK_T_X, c.m.n_layers, c.m.hidden), tr.x_out))
        assert np.array_equal(c.nxt.cpu().numpy(), N.argmax_lowest(c.logits.cpu().numpy())), t
    log(f"    multi-stream 3 steps: worst row error {worst:.3e}")
    assert worst <= TOL
