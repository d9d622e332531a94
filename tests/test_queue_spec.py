"""Pins of the reference queue builder: worked counts, the element-level static
checker, exhaustive mutation testing, and the NaN-poisoned interpreter
simulation compared with the plain forward pass."""
import json
import os
import struct

import numpy as np
import pytest

import workloads as W
from oracle import checker as CK
from oracle import numerics as N
from oracle import queue_spec as QS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SMALL = W.WORKLOADS["layer256_f32"]


def small_queue(plan=None, rows=1, ctx_max=129):
    return QS.build(SMALL.model, plan or SMALL.plan, QS.MODE_DECODE, rows, ctx_max)


def test_worked_counts_single_layer():
    g = json.load(open(os.path.join(GOLDEN, "layer256_queue_counts.json")))
    q = small_queue()
    assert len(q.instrs) == g["n_instructions"]
    counts = {}
    waits = {}
    for i, ins in enumerate(q.instrs):
        name = QS.OP_NAMES[ins.op]
        counts[name] = counts.get(name, 0) + 1
        waits.setdefault(name, set()).add(len(q.wait_list(i)))
    assert counts == g["instructions"]
    assert {k: v.pop() for k, v in waits.items() if len(v) == 1} == g["waits_per_instruction"]
    assert len(q.targets) == g["n_barriers"]
    hist = {}
    for t in q.targets:
        hist[str(t)] = hist.get(str(t), 0) + 1
    assert hist == g["targets"]
    assert sum(len(q.wait_list(i)) for i in range(len(q.instrs))) == g["n_wait_entries"]
    assert sum(q.targets) == len(q.instrs)


@pytest.mark.parametrize("name", ["layer256_f32", "llama1b_b1"])
def test_static_check_clean(name):
    wl = W.WORKLOADS[name]
    q = QS.build(wl.model, wl.plan, QS.MODE_DECODE, wl.run.batch, wl.run.ctx_max)
    assert CK.static_check(wl.model, q.parts()) == []


EDGE = [
    dict(rows=1, ctx_max=1, plan=W.Plan(tq=16, to=16, tf=32, td=16, kb=32)),     # one split, one key
    dict(rows=4, ctx_max=129, plan=W.Plan(tq=24, to=40, tf=50, td=7, kb=64)),    # ragged tiles
    dict(rows=16, ctx_max=300, plan=W.Plan(tq=512, to=256, tf=688, td=256, kb=1000)),  # one tile per op
    dict(rows=32, ctx_max=33, plan=W.Plan(tq=1, to=3, tf=5, td=9, kb=1)),        # tiny tiles, 33 splits
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: f"B{c['rows']}-ctx{c['ctx_max']}")
def test_static_check_edge_grid(case):
    q = small_queue(case["plan"], case["rows"], case["ctx_max"])
    assert CK.static_check(SMALL.model, q.parts()) == []
    assert sum(q.targets) == len(q.instrs)


def test_static_check_prefill_queue():
    m = W.ModelConfig(name="p", n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
                      ffn=96, vocab=50, rms_eps=1e-6, rope_theta=1e6, qk_norm=True)
    q = QS.build(m, W.Plan(bm=16, bn=32), QS.MODE_PREFILL, 40, 48)
    assert CK.static_check(m, q.parts()) == []
    # attention on row block m waits on the k/v tiles of row blocks 0..m only
    att = [i for i, ins in enumerate(q.instrs) if ins.op == QS.OP_P_ATTN and ins.layer == 0]
    n_waits = [len(q.wait_list(i)) for i in att]
    assert n_waits[0] < n_waits[-1]


def test_queue_does_not_depend_on_runtime_context():
    a = small_queue().parts()
    b = small_queue().parts()
    assert a == b


def test_bad_arguments_rejected():
    with pytest.raises(QS.QueueError):
        small_queue(rows=0)
    with pytest.raises(QS.QueueError):
        small_queue(rows=QS.MAX_DECODE_ROWS + 1)
    with pytest.raises(QS.QueueError):
        small_queue(plan=W.Plan(tq=0))
    with pytest.raises(QS.QueueError):
        small_queue(ctx_max=0)
    with pytest.raises(QS.QueueError):
        QS.build(SMALL.model, W.Plan(bn=48), QS.MODE_PREFILL, 8, 8)     # 48 is not whole heads of 64


# ----------------------------------------------------------------------------- mutations (every one must fail)

def _with_waits(q, i, new_list):
    """Re-encode instruction i's wait list as ranges after an edit."""
    parts = q.parts()
    p = CK.parse(parts)
    ranges = [tuple(r) for r in p.ranges.tolist()]
    recs = [list(r) for r in p.instr.tolist()]
    out_ranges = []
    for k, rec in enumerate(recs):
        lst = new_list if k == i else p.waits_of(k)
        rr = []
        for b in lst:
            if rr and rr[-1][0] + rr[-1][1] == b:
                rr[-1] = (rr[-1][0], rr[-1][1] + 1)
            else:
                rr.append((b, 1))
        rec[5], rec[6], rec[8] = len(out_ranges), len(rr), len(lst)
        out_ranges.extend(rr)
    meta = bytearray(parts["meta"])
    struct.pack_into("<I", meta, 20, len(out_ranges))
    parts = dict(parts)
    parts["meta"] = bytes(meta)
    parts["instr"] = b"".join(struct.pack("<HH7I", *r) for r in recs)
    parts["waits"] = b"".join(struct.pack("<2I", *r) for r in out_ranges)
    return parts


def test_every_single_wait_deletion_is_caught():
    q = small_queue()
    total = 0
    for i in range(len(q.instrs)):
        wl = q.wait_list(i)
        for k in range(len(wl)):
            mutant = _with_waits(q, i, wl[:k] + wl[k + 1:])
            assert CK.static_check(SMALL.model, mutant, max_errors=1), (i, k)
            total += 1
    assert total == 914


def test_every_target_decrement_is_caught():
    q = small_queue()
    parts = q.parts()
    for b in range(len(q.targets)):
        t = list(q.targets)
        t[b] -= 1
        mutant = dict(parts, targets=struct.pack(f"<{len(t)}I", *t))
        assert CK.static_check(SMALL.model, mutant, max_errors=1), b


def test_every_consumer_moved_before_a_producer_is_caught():
    q = small_queue()
    parts = q.parts()
    recs = [parts["instr"][32 * i: 32 * i + 32] for i in range(len(q.instrs))]
    sig = [ins.signal for ins in q.instrs]
    checked = 0
    for i in range(len(q.instrs)):
        producers = [j for j in range(len(q.instrs)) if sig[j] in set(q.wait_list(i))]
        if not producers:
            continue
        j = min(producers)                       # move consumer i just ahead of its first producer
        order = list(range(len(q.instrs)))
        order.remove(i)
        order.insert(j, i)
        mutant = dict(parts, instr=b"".join(recs[k] for k in order))
        assert CK.static_check(SMALL.model, mutant, max_errors=1), i
        checked += 1
    assert checked == len(q.instrs) - 32          # every instruction except the QKV tiles


# ----------------------------------------------------------------------------- simulation

def _small_inputs(ctx0=(128,), gain=0.0):
    m, r = SMALL.model, SMALL.run
    model = N.prepare(m, [W.gen.layer_weights(m, r.seed, l, gain) for l in range(m.n_layers)],
                      W.gen.global_weights(m, r.seed))
    K, V = W.gen.kv_cache(m, r)
    x0 = W.gen.input_rows(m, r)[0]
    return model, K, V, x0


@pytest.mark.parametrize("workers", [1, 2, 7, 256])
def test_simulation_matches_forward_any_schedule(workers):
    model, K, V, x0 = _small_inputs(gain=0.1)
    q = small_queue()
    parts = q.parts()
    ref = N.decode_step(model, K.copy(), V.copy(), [128], x0=x0)
    base = CK.simulate(model, parts, K.copy(), V.copy(), [128], 1, seed=0, x0=x0)
    for seed in range(100 if workers > 1 else 1):
        Ks, Vs = K.copy(), V.copy()
        res = CK.simulate(model, parts, Ks, Vs, [128], workers, seed=seed, x0=x0,
                          reverse_ties=bool(seed & 1))
        assert not res.deadlock and res.bad_reads == []
        assert np.array_equal(res.x_out, base.x_out)
        assert np.array_equal(res.counters, np.array(q.targets))
        assert not np.any(np.isnan(res.x_out))
    assert N.max_rel_err(base.x_out, ref.x_out) < 1e-12
    assert np.array_equal(Ks, base.state.K)


@pytest.mark.parametrize("ctx", [0, 1, 31, 32, 100])
def test_simulation_short_contexts_empty_splits(ctx):
    model, K, V, x0 = _small_inputs()
    q = small_queue()
    ref = N.decode_step(model, K.copy(), V.copy(), [ctx], x0=x0)
    res = CK.simulate(model, q.parts(), K.copy(), V.copy(), [ctx], 7, seed=3, x0=x0)
    assert not res.deadlock and res.bad_reads == []
    assert N.max_rel_err(res.x_out, ref.x_out) < 1e-12


def test_simulation_with_sub_queues_and_batch():
    m = SMALL.model
    plan = W.Plan(tq=16, to=16, tf=32, td=16, kb=32, n_queues=8)
    q = QS.build(m, plan, QS.MODE_DECODE, 3, 129)
    run = W.RunConfig(batch=3, ctx0=(5, 128, 64), steps=1, ctx_max=129, seed=9)
    model = N.prepare(m, [W.gen.layer_weights(m, 9, 0, 0.1)], {})
    K, V = W.gen.kv_cache(m, run)
    x0 = W.gen.input_rows(m, run)[0]
    ref = N.decode_step(model, K.copy(), V.copy(), run.ctx0, x0=x0)
    for workers in (8, 9, 64):
        res = CK.simulate(model, q.parts(), K.copy(), V.copy(), run.ctx0, workers, seed=workers, x0=x0)
        assert not res.deadlock and res.bad_reads == []
        assert N.max_rel_err(res.x_out, ref.x_out) < 1e-12


def test_simulation_detects_missing_wait():
    model, K, V, x0 = _small_inputs()
    q = small_queue()
    # drop every wait of the first O-projection tile: some schedule must read unwritten data
    i = next(k for k, ins in enumerate(q.instrs) if ins.op == QS.OP_OPROJ)
    mutant = _with_waits(q, i, [])
    seen = False
    for seed in range(20):
        res = CK.simulate(model, mutant, K.copy(), V.copy(), [128], 64, seed=seed, x0=x0)
        seen |= bool(res.bad_reads) or bool(np.any(np.isnan(res.x_out)))
    assert seen


def test_simulation_detects_deadlock():
    model, K, V, x0 = _small_inputs()
    q = small_queue()
    parts = q.parts()
    recs = [parts["instr"][32 * i: 32 * i + 32] for i in range(len(q.instrs))]
    # put the last down-projection tile first: with one worker it waits forever
    mutant = dict(parts, instr=b"".join([recs[-1]] + recs[:-1]))
    res = CK.simulate(model, mutant, K.copy(), V.copy(), [128], 1, seed=0, x0=x0)
    assert res.deadlock


# ----------------------------------------------------------------------------- fused split combines

def _fused(plan):
    import dataclasses
    return dataclasses.replace(plan, fuse_combine=1)


def test_fused_combine_queue_shape():
    """Fused: no COMBINE instructions, one barrier fewer per (layer, row, KV head),
    the O-projection waits on every split-partial tile, the META flag is set."""
    wl = W.WORKLOADS["layer256_f32"]
    m, M = wl.model, 3
    q0 = QS.build(m, wl.plan, QS.MODE_DECODE, M, 129)
    q1 = QS.build(m, _fused(wl.plan), QS.MODE_DECODE, M, 129)
    assert not any(i.op == QS.OP_COMBINE for i in q1.instrs)
    assert len(q1.instrs) == len(q0.instrs) - m.n_layers * M * m.n_kv_heads
    assert len(q1.targets) == len(q0.targets) - m.n_layers * M * m.n_kv_heads
    assert sum(q1.targets) == len(q1.instrs)
    assert struct.unpack_from("<20I", q1.meta_bytes())[19] == 1
    assert struct.unpack_from("<20I", q0.meta_bytes())[19] == 0
    oproj = next(i for i in q1.instrs if i.op == QS.OP_OPROJ)
    opart = {k for k, (t, _) in enumerate(q1.tiles) if t == QS.tensor_order(0, QS.T_OPART)}
    assert opart <= set(q1.wait_list(q1.instrs.index(oproj)))
    assert CK.static_check(m, q1.parts()) == []


@pytest.mark.parametrize("workers", [1, 7, 256])
def test_fused_combine_simulation_matches_forward(workers):
    model, K, V, x0 = _small_inputs(gain=0.1)
    wl = W.WORKLOADS["layer256_f32"]
    q = QS.build(wl.model, _fused(wl.plan), QS.MODE_DECODE, 1, 129)
    ref = N.decode_step(model, K.copy(), V.copy(), [128], x0=x0)
    base = CK.simulate(model, q.parts(), K.copy(), V.copy(), [128], 1, seed=0, x0=x0)
    assert N.max_rel_err(base.x_out, ref.x_out) < 1e-12
    for seed in range(30 if workers > 1 else 1):
        res = CK.simulate(model, q.parts(), K.copy(), V.copy(), [128], workers, seed=seed, x0=x0,
                          reverse_ties=bool(seed & 1))
        assert not res.deadlock and res.bad_reads == []
        assert np.array_equal(res.x_out, base.x_out)
        assert np.array_equal(res.counters, np.array(q.targets))


def test_fused_combine_simulation_detects_missing_split_wait():
    """Drop the O-projection's waits on the split partials (keep its residual
    wait): some schedule must read a split partial before it is written."""
    model, K, V, x0 = _small_inputs()
    wl = W.WORKLOADS["layer256_f32"]
    q = QS.build(wl.model, _fused(wl.plan), QS.MODE_DECODE, 1, 129)
    i = next(k for k, ins in enumerate(q.instrs) if ins.op == QS.OP_OPROJ)
    opart = {k for k, (t, _) in enumerate(q.tiles) if t == QS.tensor_order(0, QS.T_OPART)}
    mutant = _with_waits(q, i, [b for b in q.wait_list(i) if b not in opart])
    seen = False
    for seed in range(20):
        res = CK.simulate(model, mutant, K.copy(), V.copy(), [128], 64, seed=seed, x0=x0)
        seen |= bool(res.bad_reads) or bool(np.any(np.isnan(res.x_out)))
    assert seen
    assert CK.static_check(wl.model, mutant) != []


# ----------------------------------------------------------------------------- merge in the last split

def _merge_last(plan):
    import dataclasses
    return dataclasses.replace(plan, fuse_combine=2)


def test_merge_last_queue_shape():
    """Merge in the last split: the instructions and wait lists of the
    O-projection-fused queue, each split-partial tile's target NS + 1 (the
    splits and the merge), the META flag bit 2."""
    wl = W.WORKLOADS["layer256_f32"]
    m, M = wl.model, 3
    q1 = QS.build(m, _fused(wl.plan), QS.MODE_DECODE, M, 129)
    q2 = QS.build(m, _merge_last(wl.plan), QS.MODE_DECODE, M, 129)
    assert q2.instr_bytes() == q1.instr_bytes() and q2.waits_bytes() == q1.waits_bytes()
    opart = [k for k, (t, _) in enumerate(q2.tiles) if t == QS.tensor_order(0, QS.T_OPART)]
    assert len(opart) == M * m.n_kv_heads
    NS = q2.n_splits
    assert all(q2.targets[k] == NS + 1 for k in opart)
    assert sum(q2.targets) == len(q2.instrs) + m.n_layers * M * m.n_kv_heads
    assert struct.unpack_from("<20I", q2.meta_bytes())[19] == 4
    assert CK.static_check(m, q2.parts()) == []


def test_merge_last_every_target_change_is_caught():
    """A partial tile's target left at NS (the merge forgotten) or raised to
    NS + 2, and any other target moved by one: refused."""
    wl = W.WORKLOADS["layer256_f32"]
    q = QS.build(wl.model, _merge_last(wl.plan), QS.MODE_DECODE, 1, 129)
    parts = q.parts()
    for b in range(len(q.targets)):
        for d in (-1, 1):
            t = list(q.targets)
            t[b] += d
            mutant = dict(parts, targets=struct.pack(f"<{len(t)}I", *t))
            assert CK.static_check(wl.model, mutant, max_errors=1), (b, d)


@pytest.mark.parametrize("workers", [1, 7, 256])
def test_merge_last_simulation_matches_forward(workers):
    """Any schedule: the last split to arrive merges, the O-projection reads
    only merged rows (never a stale or unwritten element), the output equals
    the plain forward pass, counters end at their targets."""
    model, K, V, x0 = _small_inputs(gain=0.1)
    wl = W.WORKLOADS["layer256_f32"]
    q = QS.build(wl.model, _merge_last(wl.plan), QS.MODE_DECODE, 1, 129)
    ref = N.decode_step(model, K.copy(), V.copy(), [128], x0=x0)
    base = CK.simulate(model, q.parts(), K.copy(), V.copy(), [128], 1, seed=0, x0=x0)
    assert N.max_rel_err(base.x_out, ref.x_out) < 1e-12
    for seed in range(30 if workers > 1 else 1):
        res = CK.simulate(model, q.parts(), K.copy(), V.copy(), [128], workers, seed=seed, x0=x0,
                          reverse_ties=bool(seed & 1))
        assert not res.deadlock and res.bad_reads == []
        assert np.array_equal(res.x_out, base.x_out)
        assert np.array_equal(res.counters, np.array(q.targets))


def test_merge_last_simulation_detects_early_merge_and_missing_wait():
    """Target NS (the last split taken to be the one before it): the merge
    reads a partial not yet written.  O-projection without its partial-tile
    waits: it reads attention rows not yet merged."""
    model, K, V, x0 = _small_inputs()
    wl = W.WORKLOADS["layer256_f32"]
    q = QS.build(wl.model, _merge_last(wl.plan), QS.MODE_DECODE, 1, 129)
    opart = {k for k, (t, _) in enumerate(q.tiles) if t == QS.tensor_order(0, QS.T_OPART)}
    t = [v - 1 if k in opart else v for k, v in enumerate(q.targets)]
    early = dict(q.parts(), targets=struct.pack(f"<{len(t)}I", *t))
    i = next(k for k, ins in enumerate(q.instrs) if ins.op == QS.OP_OPROJ)
    nowait = _with_waits(q, i, [b for b in q.wait_list(i) if b not in opart])
    for mutant in (early, nowait):
        seen = False
        for seed in range(20):
            res = CK.simulate(model, mutant, K.copy(), V.copy(), [128], 64, seed=seed, x0=x0)
            seen |= bool(res.bad_reads) or bool(np.any(np.isnan(res.x_out)))
        assert seen
        assert CK.static_check(wl.model, mutant) != []


def test_attention_splits_are_split_major_and_rotated():
    """Hand-worked order for 3 rows x 2 KV heads x 3 splits: split s starts at
    the pair s rows on and wraps, so a worker taking every n-th instruction by
    position meets several rows."""
    q = QS.build(W.LLAMA_LAYER_F32, W.Plan(tq=16, to=16, tf=32, td=16, kb=32), QS.MODE_DECODE, 3, 96)
    att = [(i.a0, i.a1, i.a2) for i in q.instrs if i.op == QS.OP_ATTN]
    assert att == [(0, 0, 0), (0, 1, 0), (1, 0, 0), (1, 1, 0), (2, 0, 0), (2, 1, 0),
                   (1, 0, 1), (1, 1, 1), (2, 0, 1), (2, 1, 1), (0, 0, 1), (0, 1, 1),
                   (2, 0, 2), (2, 1, 2), (0, 0, 2), (0, 1, 2), (1, 0, 2), (1, 1, 2)]


# ----------------------------------------------------------------------------- loop queues (multi-step decode)

TINY = W.ModelConfig("tiny-loop", n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, ffn=96,
                     vocab=200, rms_eps=1e-5, rope_theta=1e4)
TINY_PLAN = W.Plan(tq=16, to=16, tf=32, td=16, kb=8, loop=1)
TINY_RUN = W.RunConfig(batch=2, ctx0=(9, 13), steps=3, ctx_max=20, seed=21)


def _tiny(plan=TINY_PLAN):
    q = QS.build(TINY, plan, QS.MODE_DECODE, TINY_RUN.batch, TINY_RUN.ctx_max)
    model = N.prepare(TINY, W.gen.all_layer_weights(TINY, TINY_RUN.seed, 0.1),
                      W.gen.global_weights(TINY, TINY_RUN.seed, 0.1))
    K, V = W.gen.kv_cache(TINY, TINY_RUN)
    return q, model, K, V, W.gen.decode_tokens(TINY, TINY_RUN)


def test_loop_queue_shape():
    """One step of a loop queue: the single-step queue, then ceil(V / 64) LM-head
    tiles and one argmax per row; every embedding tile waits (flagged as the
    previous step's) on all argmax barriers, in one range."""
    import dataclasses
    q, *_ = _tiny()
    q1 = QS.build(TINY, dataclasses.replace(TINY_PLAN, loop=0), QS.MODE_DECODE, 2, 20)
    nV = -(-TINY.vocab // QS.LM_TILE)
    assert len(q.instrs) == len(q1.instrs) + nV + 2
    assert [i.op for i in q.instrs[len(q1.instrs):]] == [QS.OP_LMHEAD] * nV + [QS.OP_ARGMAX] * 2
    assert q.flags == 2 and q1.flags == 0
    next_ids = [q.instrs[-2].signal, q.instrs[-1].signal]
    for ins in q.instrs:
        if ins.op == QS.OP_EMBED:
            assert q.waits[ins.wait_off: ins.wait_off + ins.wait_cnt] == [(next_ids[0], 2 | QS.PREV)]
            assert q.wait_list(ins_index := q.instrs.index(ins)) == []
            assert q.wait_list(ins_index, prev=True) == next_ids
    lm = [i for i in q.instrs if i.op == QS.OP_LMHEAD]
    assert [(i.a0, i.a1) for i in lm] == [(0, 64), (64, 128), (128, 192), (192, 200)]
    assert sum(q.targets) == len(q.instrs)
    assert CK.static_check(TINY, q.parts()) == []


def test_loop_queue_refused_without_embedding_or_lm_head():
    import dataclasses
    with pytest.raises(QS.QueueError):
        QS.build(W.LLAMA_LAYER_F32, dataclasses.replace(SMALL.plan, loop=1), QS.MODE_DECODE, 1, 129)
    with pytest.raises(QS.QueueError):
        QS.build(TINY, TINY_PLAN, QS.MODE_PREFILL, 16, 20)


def _with_ranges(parts, i, ranges):
    """Replace instruction i's wait ranges (re-encoding every record's offsets)."""
    p = CK.parse(parts)
    recs = [list(r) for r in p.instr.tolist()]
    out = []
    for k, rec in enumerate(recs):
        rr = ranges if k == i else [tuple(x) for x in p.ranges[rec[5]: rec[5] + rec[6]].tolist()]
        rec[5], rec[6] = len(out), len(rr)
        rec[8] = sum(c & ~QS.PREV for _, c in rr)
        out.extend(rr)
    meta = bytearray(parts["meta"])
    struct.pack_into("<I", meta, 20, len(out))
    return dict(parts, meta=bytes(meta), instr=b"".join(struct.pack("<HH7I", *r) for r in recs),
                waits=b"".join(struct.pack("<2I", *r) for r in out))


def test_loop_every_single_wait_deletion_is_caught():
    """Exhaustive on the tiny loop queue, previous-step waits included."""
    q, *_ = _tiny()
    parts = q.parts()
    total = 0
    for i in range(len(q.instrs)):
        for prev in (False, True):
            wl = q.wait_list(i, prev=prev)
            other = [(f, c) for f, c in q.waits[q.instrs[i].wait_off: q.instrs[i].wait_off + q.instrs[i].wait_cnt]
                     if bool(c & QS.PREV) != prev]
            for k in range(len(wl)):
                keep = wl[:k] + wl[k + 1:]
                rr = [(b, 1 | (QS.PREV if prev else 0)) for b in keep]
                mutant = _with_ranges(parts, i, (other + rr) if prev else (rr + other))
                assert CK.static_check(TINY, mutant, max_errors=1), (i, prev, k)
                total += 1
    assert total == sum(i.n_wait for i in q.instrs)


def test_loop_previous_step_flag_is_checked():
    """An embedding tile whose argmax waits lose the previous-step flag waits on
    producers later in the queue: refused (it could never start)."""
    q, *_ = _tiny()
    i = next(k for k, ins in enumerate(q.instrs) if ins.op == QS.OP_EMBED)
    f, c = q.waits[q.instrs[i].wait_off]
    mutant = _with_ranges(q.parts(), i, [(f, c & ~QS.PREV)])
    assert any("not earlier" in e for e in CK.static_check(TINY, mutant))


@pytest.mark.parametrize("workers", [1, 2, 7, 64])
def test_loop_simulation_teacher_forced_matches_oracle(workers):
    """Three steps in one run, any schedule: every step's logits equal the
    oracle's teacher-forced step (float64, same tile bodies) and are identical
    across schedules; counters end at 3 x targets; the cache holds all steps."""
    q, model, K, V, tokens = _tiny()
    parts = q.parts()
    Kr, Vr = K.copy(), V.copy()
    ref = [N.decode_step(model, Kr, Vr, [p + t for p in TINY_RUN.ctx0], tokens=tokens[t]) for t in range(3)]
    base = None
    for seed in range(25 if workers > 1 else 1):
        Ks, Vs = K.copy(), V.copy()
        res = CK.simulate(model, parts, Ks, Vs, TINY_RUN.ctx0, workers, seed=seed, tokens=tokens[:3],
                          steps=3, reverse_ties=bool(seed & 1))
        assert not res.deadlock and res.bad_reads == []
        assert np.array_equal(res.counters, 3 * np.array(q.targets))
        got = [res.state.logits[t] for t in range(3)]
        for t in range(3):
            assert N.max_rel_err_rows(got[t], ref[t].logits) < 1e-12
            assert np.array_equal(res.state.next[t], N.argmax_lowest(got[t]))
        if base is None:
            base = got
        assert all(np.array_equal(a, b) for a, b in zip(base, got))
        assert np.array_equal(Ks, Kr) and np.array_equal(Vs, Vr)


def test_loop_merge_last_simulation_matches_oracle():
    """Loop queue whose last split merges: at step t the last arrival sees
    (NS + 1) t + NS - 1 earlier signals; three steps in one run equal the
    oracle's teacher-forced steps and the counters end at 3 x targets."""
    import dataclasses
    q, model, K, V, tokens = _tiny(dataclasses.replace(TINY_PLAN, fuse_combine=2))
    assert CK.static_check(TINY, q.parts()) == []
    Kr, Vr = K.copy(), V.copy()
    ref = [N.decode_step(model, Kr, Vr, [p + t for p in TINY_RUN.ctx0], tokens=tokens[t]) for t in range(3)]
    for seed in range(10):
        res = CK.simulate(model, q.parts(), K.copy(), V.copy(), TINY_RUN.ctx0, 7, seed=seed, tokens=tokens[:3],
                          steps=3, reverse_ties=bool(seed & 1))
        assert not res.deadlock and res.bad_reads == []
        assert np.array_equal(res.counters, 3 * np.array(q.targets))
        for t in range(3):
            assert N.max_rel_err_rows(res.state.logits[t], ref[t].logits) < 1e-12


def test_loop_simulation_greedy_feedback():
    """With the argmax fed back, step t + 1 embeds step t's argmax: the same as
    teacher-forcing with that chain of tokens."""
    q, model, K, V, tokens = _tiny()
    res = CK.simulate(model, q.parts(), K.copy(), V.copy(), TINY_RUN.ctx0, 7, seed=5, tokens=tokens[:1],
                      steps=3, feedback=True)
    assert not res.deadlock and res.bad_reads == []
    chain = [tokens[0], res.state.next[0], res.state.next[1]]
    Kr, Vr = K.copy(), V.copy()
    for t in range(3):
        tr = N.decode_step(model, Kr, Vr, [p + t for p in TINY_RUN.ctx0], tokens=chain[t])
        assert N.max_rel_err_rows(res.state.logits[t], tr.logits) < 1e-12
        assert np.array_equal(res.state.next[t], N.argmax_lowest(tr.logits))


def test_loop_simulation_detects_missing_previous_step_wait():
    """Embedding tiles that do not wait for the previous step's argmax: some
    schedule overwrites X_0 while the previous step still reads it, or embeds
    a token that is not yet there."""
    q, model, K, V, tokens = _tiny()
    parts = q.parts()
    for i, ins in enumerate(q.instrs):
        if ins.op == QS.OP_EMBED:
            parts = _with_ranges(parts, i, [])
    assert CK.static_check(TINY, parts) != []
    seen = False
    for seed in range(20):
        res = CK.simulate(model, parts, K.copy(), V.copy(), TINY_RUN.ctx0, 64, seed=seed, tokens=tokens[:1],
                          steps=3, feedback=True)
        seen |= bool(res.bad_reads)
    assert seen
