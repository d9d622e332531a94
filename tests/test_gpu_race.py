"""Race checks of the tile hand-off on the GPU, and the trace mode.

The hand-off stores intermediate tiles with agent-scope (device-coherent)
stores, waits for their acknowledgement, then bumps the tile's counter; a
consumer polls the counters of exactly the tiles it reads.  Two checks widen
any window in which a consumer could read a tile before its producer wrote it:

* poison: every byte of the workspace is set to 0xFF before the step, so every
  intermediate float starts as NaN (counters and queue heads are cleared by the
  step itself); a tile read too early carries NaN into the outputs;
* delay injection (MK_OPT_DELAY_SEED): each producer stalls for a seeded
  pseudo-random 0..50 us before it stores its tile.

Each poisoned, delayed run must give outputs bit-identical to a clean run, with
no NaN, and the counters must end at their targets.  The runs cover the fp32
layer and a two-layer 1B-shaped model, with one static sub-queue per worker,
with shared sub-queues (dynamic pops) and with the attention splits handed out
at run time, and the prefill interpreter.  A stress
run stops at its first failure.
"""
import dataclasses

import numpy as np
import pytest
import torch

import tile_synchronized_decoder_amd as T
from tile_synchronized_decoder_amd import trace as TR
import workloads as W

pytestmark = pytest.mark.gpu

SEEDS = (1, 2, 3)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _decode_cases():
    ncu = 256
    f32 = W.WORKLOADS["layer256_f32"]
    base = W.shrink(W.WORKLOADS["llama1b_b1"], n_layers=2, vocab=4096, batch=1, ctx0=(1024,), steps=1)
    b4 = W.shrink(W.WORKLOADS["llama1b_b1"], n_layers=2, vocab=4096, batch=4, ctx0=(1024, 37, 600, 1),
                  steps=1, name="llama1b_L2_B4")
    b6 = W.shrink(W.WORKLOADS["llama1b_b1"], n_layers=2, vocab=4096, batch=6, ctx0=(1024, 37, 600, 1, 300, 900),
                  steps=1, name="llama1b_L2_B6")
    return {
        "f32_layer_static": dataclasses.replace(f32, plan=dataclasses.replace(f32.plan, n_queues=ncu)),
        "f32_layer_shared8": dataclasses.replace(f32, plan=dataclasses.replace(f32.plan, n_queues=8)),
        "bf16_1b_b1_static": dataclasses.replace(base, plan=W.Plan(tf=32, td=8, n_queues=ncu)),
        "bf16_1b_b4_shared8": dataclasses.replace(b4, plan=W.Plan(n_queues=8)),
        "bf16_1b_b1_fused_static": dataclasses.replace(base, plan=W.Plan(tf=32, td=8, n_queues=ncu,
                                                                         fuse_combine=1)),
        # splits handed out at run time (ragged contexts, 128-key splits), with
        # split combines and with the merge in the last split
        "bf16_1b_b6_attn_pop": dataclasses.replace(b6, plan=W.Plan(tf=32, td=8, kb=128, n_queues=ncu, attn_pop=1)),
        "bf16_1b_b6_attn_pop_merge": dataclasses.replace(b6, plan=W.Plan(tf=32, td=8, kb=128, n_queues=ncu,
                                                                         attn_pop=1, fuse_combine=2)),
    }


def _outputs(c):
    """Every intermediate tensor of the step, the logits and argmax, the new cache entries."""
    m = c.m
    fused = c.wl.plan.fuse_combine
    out = {f"x{l}": c.tensor(T.MK_T_X, l, m.hidden) for l in range(m.n_layers + 1)}
    for l in range(m.n_layers):
        out[f"qkv{l}"] = c.tensor(T.MK_T_QKV, l, m.qkv_cols)
        if not fused:
            out[f"att{l}"] = c.tensor(T.MK_T_ATT, l, m.attn_cols)
        out[f"h{l}"] = c.tensor(T.MK_T_HRES, l, m.hidden)
        out[f"act{l}"] = c.tensor(T.MK_T_ACT, l, m.ffn)
    if c.logits is not None:
        out["logits"] = c.logits.cpu().numpy().copy()
        out["next"] = c.nxt.cpu().numpy().copy()
    k, v = c.kv_host()
    out["k"], out["v"] = k.copy(), v.copy()
    return out


def _run(c, ctx, poison: bool, seed: int):
    c.reset_kv()
    if poison:
        c.ws.fill_(255)
        if c.logits is not None:
            c.logits.fill_(float("nan"))
            c.nxt.fill_(-1)
    T.mk_set_option(T.MK_OPT_DELAY_SEED, seed)
    try:
        c.step(0, ctx, T.MK_MEGAKERNEL)
    finally:
        T.mk_set_option(T.MK_OPT_DELAY_SEED, 0)
    err = T.mk_device_error(c.q, c.ws)
    assert err.code == 0, (err.code, err.instr, err.barrier, err.value, err.target)
    tg = np.frombuffer(c.q.export(T.MK_PART_TARGETS), dtype=np.uint32)
    assert np.array_equal(c.counters(), tg), "counters must end at their targets"
    return _outputs(c)


@pytest.mark.parametrize("name", list(_decode_cases()))
def test_decode_poisoned_and_delayed_runs_are_bit_identical(name):
    from _gpucase import make_case, log
    wl = _decode_cases()[name]
    c = make_case(wl, gain_jitter=0.1)
    ctx = list(wl.run.ctx0)
    clean = _run(c, ctx, poison=False, seed=0)
    for k, v in clean.items():
        if v.dtype.kind == "f":
            assert np.isfinite(v).all(), k
    for seed in SEEDS:
        got = _run(c, ctx, poison=True, seed=seed)
        bad = [k for k in clean if not np.array_equal(clean[k], got[k])]
        log(f"    {name} seed {seed}: {'identical' if not bad else 'DIFFERS in ' + ','.join(bad[:6])}")
        assert not bad, bad


def test_prefill_poisoned_and_delayed_runs_are_bit_identical():
    """The prefill interpreter (one shared sub-queue and eight), S = 200 over
    two row blocks: outputs of poisoned, delayed runs equal a clean run."""
    from _gpucase import log
    from test_gpu_prefill import SMALL, PrefillCase
    c = PrefillCase(SMALL, s_max=256, ctx_max=320, kv_rows=1, seed=5)
    S = 200
    for nq in (1, 8):
        c.q = T.mk_build_queue(T.make_config(SMALL), T.make_plan(W.Plan(n_queues=nq), T.MK_PREFILL, 256, 320))
        from tile_synchronized_decoder_amd import device as D
        c.dq, c.ws = D.upload_queue(c.q), D.workspace(c.q)
        results = []
        for seed in (0,) + SEEDS:
            c.reset()
            if seed:
                c.ws.fill_(255)
                c.logits.fill_(float("nan"))
            T.mk_set_option(T.MK_OPT_DELAY_SEED, seed)
            try:
                c.prefill(S, 0, T.MK_MEGAKERNEL)
            finally:
                T.mk_set_option(T.MK_OPT_DELAY_SEED, 0)
            results.append(c.snapshot(S))
        for k, v in results[0].items():
            if v.dtype.kind == "f":
                assert np.isfinite(v).all(), k
        for seed, got in zip(SEEDS, results[1:]):
            bad = [k for k in results[0] if not np.array_equal(results[0][k], got[k])]
            log(f"    prefill n_queues={nq} seed {seed}: {'identical' if not bad else 'DIFFERS ' + ','.join(bad[:6])}")
            assert not bad, bad


# ----------------------------------------------------------------------------- trace mode

_INSTR = np.dtype([("op", "<u2"), ("layer", "<u2"), ("a0", "<u4"), ("a1", "<u4"), ("a2", "<u4"),
                   ("wait_off", "<u4"), ("wait_cnt", "<u4"), ("signal", "<u4"), ("n_wait", "<u4")])


@pytest.mark.parametrize("n_queues", [256, 8])
def test_trace_records_every_instruction_once_in_order(n_queues):
    """Trace mode on a two-layer 1B-shaped step: every instruction has one
    record from one worker; pop <= waits ended <= end; a worker's instructions
    do not overlap in time; every producer of a waited tile was popped before
    its consumer's wait ended; traced results equal untraced ones."""
    from _gpucase import make_case, log
    wl = W.shrink(W.WORKLOADS["llama1b_b1"], n_layers=2, vocab=4096, batch=2, ctx0=(1024, 300), steps=1)
    wl = dataclasses.replace(wl, plan=W.Plan(tf=32, td=8, n_queues=n_queues))
    c = make_case(wl)
    ctx = list(wl.run.ctx0)
    c.reset_kv()
    c.step(0, ctx, T.MK_MEGAKERNEL)
    ref = _outputs(c)
    instr = np.frombuffer(c.q.export(T.MK_PART_INSTR), dtype=_INSTR)
    waits = np.frombuffer(c.q.export(T.MK_PART_WAITS), dtype=np.uint32).reshape(-1, 2)
    n = len(instr)
    buf = torch.zeros(8 * n, dtype=torch.int64, device="cuda")
    T.mk_set_option(T.MK_OPT_TRACE_BYTES, buf.numel() * 8)
    T.mk_set_option(T.MK_OPT_TRACE_BUFFER, buf.data_ptr())
    try:
        c.reset_kv()
        c.step(0, ctx, T.MK_MEGAKERNEL)
    finally:
        T.mk_set_option(T.MK_OPT_TRACE_BUFFER, 0)
        T.mk_set_option(T.MK_OPT_TRACE_BYTES, 0)
    assert T.mk_device_error(c.q, c.ws).code == 0
    got = _outputs(c)
    assert all(np.array_equal(ref[k], got[k]) for k in ref), "tracing changed the results"
    raw = buf.cpu().numpy().view(np.uint64).reshape(n, 8)
    assert (raw[:, 1] > 0).all() and (raw[:, 5] > 0).all(), "an instruction left no record"
    assert (raw[:, 6] == 0).all() and (raw[:, 7] == 0).all()
    rec = TR.parse(raw.reshape(-1), c.q.export(T.MK_PART_INSTR))
    ncu = T.mk_get_option(T.MK_OPT_NUM_CUS)
    assert ((rec["wg"] >= 0) & (rec["wg"] < ncu)).all()
    assert (rec["xcd"] < 8).all()
    assert (rec["start"] <= rec["ready"]).all() and (rec["ready"] <= rec["end"]).all()
    if n_queues == ncu:
        # static assignment: instruction i runs on worker i mod n_queues
        assert np.array_equal(rec["wg"], np.arange(n) % n_queues)
    # one instruction at a time per worker
    for wg in np.unique(rec["wg"]):
        r = np.sort(rec[rec["wg"] == wg], order="start")
        assert (r["end"][:-1] <= r["start"][1:]).all(), f"worker {wg} overlaps"
    # every producer of a waited barrier was popped before the consumer's wait ended
    writers = {}
    for i, s in enumerate(instr["signal"]):
        writers.setdefault(int(s), []).append(i)
    checked = 0
    for i in range(n):
        for k in range(int(instr["wait_off"][i]), int(instr["wait_off"][i] + instr["wait_cnt"][i])):
            first, cnt = waits[k]
            for bar in range(int(first), int(first + cnt)):
                for p in writers[bar]:
                    assert rec["start"][p] <= rec["ready"][i], (i, p, bar)
                    checked += 1
    # each waited barrier was checked against all of its writers (the attention-split
    # partials have one writer per split)
    assert checked >= int(instr["n_wait"].astype(np.int64).sum())
    stats = TR.op_stats(rec)
    log(f"    trace n_queues={n_queues}: {n} instructions, {checked} producer->consumer pairs; "
        + ", ".join(f"{k} wait {v['wait_us']:.1f} us" for k, v in stats.items()))
