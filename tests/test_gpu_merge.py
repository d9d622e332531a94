"""Split partials merged by the last-arriving split (plan fuse_combine = 2) on the GPU.

The queue has no COMBINE instructions: every attention split counts its
arrival on its (row, KV head) partial tile, the split whose arrival completes
the count merges the partials into the attention output with the combine's
own code, and signals the tile once more.  The merge reads the partials in the
same order as a COMBINE tile, so every output (each layer's intermediates, the
new cache entries, logits, argmax) must equal a queue with COMBINE tiles bit
for bit, in every execution mode, also with a NaN-poisoned workspace and
seeded producer delays, and over several steps of one persistent launch.
"""
import dataclasses

import numpy as np
import pytest
import torch

import tile_synchronized_decoder_amd as T
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(autouse=True)
def _restore_options():
    yield
    T.mk_set_option(T.MK_OPT_DELAY_SEED, 0)
    T.mk_set_option(T.MK_OPT_STREAMS, 2)


def _cases():
    ncu = 256
    f32 = W.WORKLOADS["layer256_f32"]
    f32_b3 = W.shrink(f32, batch=3, ctx0=(128, 0, 31), name="layer256_f32_b3")
    b1 = W.shrink(W.WORKLOADS["llama1b_b1"], n_layers=2, vocab=4096, batch=1, ctx0=(1024,), steps=1)
    b4 = W.shrink(W.WORKLOADS["llama1b_b1"], n_layers=2, vocab=4096, batch=4, ctx0=(1024, 37, 600, 1),
                  steps=1, name="llama1b_L2_B4")
    e8 = W.shrink(W.WORKLOADS["llama8b_b1"], n_layers=2, vocab=4096, steps=1, name="llama8b_L2_B1")
    return {
        "f32_layer": f32,
        "f32_layer_b3_short": dataclasses.replace(f32_b3, plan=dataclasses.replace(f32.plan, n_queues=8)),
        "bf16_1b_b1_static": dataclasses.replace(b1, plan=W.Plan(tf=32, td=8, n_queues=ncu)),
        "bf16_1b_b4_shared8": dataclasses.replace(b4, plan=W.Plan(n_queues=8)),
        "bf16_8b_b1_static": e8,
    }


def _with_fuse(wl, fuse):
    return dataclasses.replace(wl, plan=dataclasses.replace(wl.plan, fuse_combine=fuse))


def _outputs(c):
    m = c.m
    out = {f"x{l}": c.tensor(T.MK_T_X, l, m.hidden) for l in range(m.n_layers + 1)}
    for l in range(m.n_layers):
        out[f"qkv{l}"] = c.tensor(T.MK_T_QKV, l, m.qkv_cols)
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
    # every mode counts the split arrivals; the megakernel and multi-stream modes count every tile
    tg = np.frombuffer(c.q.export(T.MK_PART_TARGETS), dtype=np.uint32)
    got = c.counters()
    if mode in (T.MK_MEGAKERNEL, T.MK_MULTI_STREAM):
        assert np.array_equal(got, tg), "counters must end at their targets"
    else:
        opart = tg > 1
        assert np.array_equal(got[opart], tg[opart]), "split arrivals plus merges must reach the targets"
    return _outputs(c)


def _diff(a, b):
    return [k for k in a if not np.array_equal(a[k], b[k])]


@pytest.mark.parametrize("name", list(_cases()))
def test_merge_last_equals_combine_tiles_bitwise(name):
    from _gpucase import make_case, log
    wl = _cases()[name]
    ref = _run(make_case(_with_fuse(wl, 0), gain_jitter=0.1), T.MK_MEGAKERNEL)
    for k, v in ref.items():
        if v.dtype.kind == "f":
            assert np.isfinite(v).all(), k
    c = make_case(_with_fuse(wl, 2), gain_jitter=0.1)
    for label, mode in (("mega", T.MK_MEGAKERNEL), ("kpo", T.MK_KERNEL_PER_OP),
                        ("kpo_graph", T.MK_KERNEL_PER_OP_GRAPH), ("kpo_graph_replay", T.MK_KERNEL_PER_OP_GRAPH),
                        ("multi_stream", T.MK_MULTI_STREAM)):
        bad = _diff(ref, _run(c, mode))
        log(f"    {name} {label}: {'identical' if not bad else 'DIFFERS in ' + ','.join(bad[:6])}")
        assert not bad, (label, bad)


@pytest.mark.parametrize("name", ["bf16_1b_b1_static", "bf16_1b_b4_shared8", "bf16_8b_b1_static"])
def test_merge_last_poisoned_and_delayed_runs_are_bit_identical(name):
    from _gpucase import make_case, log
    c = make_case(_with_fuse(_cases()[name], 2), gain_jitter=0.1)
    clean = _run(c, T.MK_MEGAKERNEL)
    for mode, seed in ((T.MK_MEGAKERNEL, 1), (T.MK_MEGAKERNEL, 2), (T.MK_MULTI_STREAM, 3)):
        bad = _diff(clean, _run(c, mode, poison=True, seed=seed))
        log(f"    {name} mode {mode} seed {seed}: {'identical' if not bad else 'DIFFERS in ' + ','.join(bad[:6])}")
        assert not bad, (mode, seed, bad)


def test_merge_last_loop_equals_combine_loop():
    """Four steps in one persistent launch (the arrival count of step t starts
    at (NS + 1) t): logits, argmax and last hidden rows equal the loop queue
    with COMBINE tiles bit for bit, also poisoned and delayed."""
    from _gpucase import make_case
    from test_gpu_loop import _case, _run_loop, STEPS
    ref_c = _case(2, (1000, 333), 8)
    ref = _run_loop(ref_c, ref_c.tokens[:STEPS], feedback=1)
    c = make_case(_with_fuse(ref_c.wl, 2), gain_jitter=0.1)
    got = _run_loop(c, c.tokens[:STEPS], feedback=1)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
    c.ws.fill_(255)
    T.mk_set_option(T.MK_OPT_DELAY_SEED, 5)
    try:
        got = _run_loop(c, c.tokens[:STEPS], feedback=1)
    finally:
        T.mk_set_option(T.MK_OPT_DELAY_SEED, 0)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
