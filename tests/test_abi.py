"""The C ABI library on the CPU: it loads, exports every entry point that
include/mk.h declares, and its host-side queue builder (an independent C++
implementation) produces the reference builder's bytes exactly."""
import ctypes
import dataclasses
import os
import re

import numpy as np
import pytest

import tile_synchronized_decoder_amd as T
from tile_synchronized_decoder_amd import _lib as L
import workloads as W
from oracle import queue_spec as QS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "mk.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    syms = declared_symbols()
    assert len(syms) >= 13
    for s in syms:
        assert hasattr(lib, s), s
    assert sorted(L.EXPORTED) == syms


def _both(model, plan, mode, rows, ctx_max):
    q = T.mk_build_queue(T.make_config(model), T.make_plan(plan, mode, rows, ctx_max))
    return q.parts(), QS.build(model, plan, mode, rows, ctx_max).parts()


@pytest.mark.parametrize("name", ["layer256_f32", "llama1b_b1", "llama8b_b1", "llama8b_b4",
                                  "llama1b_stream_b32"])
def test_builder_bytes_equal_reference(name):
    wl = W.WORKLOADS[name]
    got, ref = _both(wl.model, wl.plan, QS.MODE_DECODE, wl.run.batch, wl.run.ctx_max)
    for part in ref:
        assert got[part] == ref[part], part


EDGE = [
    (1, 1, W.Plan(tq=16, to=16, tf=32, td=16, kb=32)),
    (4, 129, W.Plan(tq=24, to=40, tf=50, td=7, kb=64)),
    (16, 300, W.Plan(tq=512, to=256, tf=688, td=256, kb=1000)),
    (32, 33, W.Plan(tq=1, to=3, tf=5, td=9, kb=1)),
    (3, 129, W.Plan(tq=16, to=16, tf=32, td=16, kb=32, n_queues=8)),
]


@pytest.mark.parametrize("rows,ctx,plan", EDGE)
def test_builder_bytes_edge_grid(rows, ctx, plan):
    got, ref = _both(W.LLAMA_LAYER_F32, plan, QS.MODE_DECODE, rows, ctx)
    assert got == ref


def test_builder_bytes_gqa_one_kv_head():
    m = W.ModelConfig(name="mqa", n_layers=2, hidden=128, n_q_heads=4, n_kv_heads=1, head_dim=64,
                      ffn=96, vocab=10, rms_eps=1e-5, rope_theta=1e4)
    got, ref = _both(m, W.Plan(tq=48, to=16, tf=32, td=16, kb=16), QS.MODE_DECODE, 2, 40)
    assert got == ref


@pytest.mark.parametrize("S,bm,bn", [(40, 16, 32), (64, 64, 64), (17, 8, 96)])
def test_builder_bytes_prefill(S, bm, bn):
    m = W.ModelConfig(name="p", n_layers=2, hidden=96, n_q_heads=4, n_kv_heads=2, head_dim=32,
                      ffn=160, vocab=50, rms_eps=1e-6, rope_theta=1e6, qk_norm=True)
    got, ref = _both(m, W.Plan(bm=bm, bn=bn), QS.MODE_PREFILL, S, 64)
    assert got == ref


def test_builder_bytes_prefill_qwen_shape():
    wl = W.WORKLOADS["qwen8b_prefill"]
    m = W.shrink(wl, n_layers=2).model
    got, ref = _both(m, wl.plan, QS.MODE_PREFILL, 512, wl.run.ctx_max)
    assert got == ref
    got, ref = _both(m, wl.plan.for_prefill(), QS.MODE_PREFILL, 512, wl.run.ctx_max)   # its own sub-queues
    assert got == ref


@pytest.mark.parametrize("kw", [dict(rows=0), dict(rows=33), dict(ctx_max=0), dict(tq=0), dict(kb=0),
                                dict(n_queues=0), dict(n_queues=1025)])
def test_builder_rejects_what_the_reference_rejects(kw):
    plan = W.Plan(**{k: v for k, v in kw.items() if k in ("tq", "kb", "n_queues")})
    rows = kw.get("rows", 1)
    ctx = kw.get("ctx_max", 10)
    with pytest.raises(QS.QueueError):
        QS.build(W.LLAMA_LAYER_F32, plan, QS.MODE_DECODE, rows, ctx)
    with pytest.raises(L.MkError) as e:
        T.mk_build_queue(T.make_config(W.LLAMA_LAYER_F32), T.make_plan(plan, QS.MODE_DECODE, rows, ctx))
    assert e.value.status == L.MK_EINVAL


def test_prefill_rejects_partial_heads():
    with pytest.raises(L.MkError):
        T.mk_build_queue(T.make_config(W.LLAMA_LAYER_F32), T.make_plan(W.Plan(bn=48), QS.MODE_PREFILL, 8, 8))


def test_workspace_layout_is_consistent():
    wl = W.WORKLOADS["llama1b_b1"]
    q = T.mk_build_queue(T.make_config(wl.model), T.make_plan(wl.plan, 0, 1, wl.run.ctx_max))
    total = q.workspace_nbytes()
    offs = [q.workspace_offset(T.MK_T_X, l) for l in range(17)]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert q.workspace_offset(T.MK_T_ERROR) < total
    with pytest.raises(L.MkError):
        q.workspace_offset(T.MK_T_QKV, 16)


@pytest.mark.parametrize("fuse", [1, 2])
@pytest.mark.parametrize("rows,ctx,plan", [
    (1, 129, W.Plan(tq=16, to=16, tf=32, td=16, kb=32)),
    (3, 129, W.Plan(tq=24, to=40, tf=50, td=7, kb=64, n_queues=8)),
    (32, 33, W.Plan(tq=1, to=3, tf=5, td=9, kb=1)),
])
def test_builder_bytes_fused_combine(rows, ctx, plan, fuse):
    """Queues without split-combine instructions (merged in the O-projection,
    or by the last-arriving split): byte-identical."""
    got, ref = _both(W.LLAMA_LAYER_F32, dataclasses.replace(plan, fuse_combine=fuse), QS.MODE_DECODE, rows, ctx)
    assert got == ref


@pytest.mark.parametrize("name,fuse,loop", [("llama1b_b1", 1, 0), ("llama1b_b1", 2, 0), ("llama8b_b1", 2, 0),
                                            ("llama1b_b1", 2, 1)])
def test_builder_bytes_fused_combine_full_shapes(name, fuse, loop):
    wl = W.WORKLOADS[name]
    plan = dataclasses.replace(wl.plan, fuse_combine=fuse, loop=loop)
    got, ref = _both(wl.model, plan, QS.MODE_DECODE, wl.run.batch, wl.run.ctx_max)
    assert got == ref


@pytest.mark.parametrize("fuse", [-1, 3])
def test_builder_rejects_bad_fuse_flag(fuse):
    wl = W.WORKLOADS["layer256_f32"]
    plan = dataclasses.replace(wl.plan, fuse_combine=fuse)
    with pytest.raises(T.MkError):
        T.mk_build_queue(T.make_config(wl.model), T.make_plan(plan, QS.MODE_DECODE, 1, 129))
    with pytest.raises(QS.QueueError):
        QS.build(wl.model, plan, QS.MODE_DECODE, 1, 129)


def test_options_validate_and_round_trip():
    """Process-wide options are host state: out-of-range values are refused
    (status, no change), valid ones read back."""
    for key, good, bad in ((T.MK_OPT_GEMV_PIPE, (0, 1, 2), (-1, 3)),
                           (T.MK_OPT_WORKERS_PER_CU, (1, 2), (0, 9)),
                           (T.MK_OPT_SPIN_LIMIT, (1, 1 << 20), (0,)),
                           (T.MK_OPT_DELAY_SEED, (0, 7, 0xFFFFFFFF), (-1, 1 << 32)),
                           (T.MK_OPT_STREAMS, (1, 8, 2), (0, 9)),
                           (T.MK_OPT_MEGAKERNELS, (2, 8, 1), (0, 9)),
                           (T.MK_OPT_PREFILL_LO, (0, 7, 15), (-1, 16))):
        old = T.mk_get_option(key)
        try:
            for v in good:
                T.mk_set_option(key, v)
                assert T.mk_get_option(key) == v
            for v in bad:
                with pytest.raises(T.MkError):
                    T.mk_set_option(key, v)
                assert T.mk_get_option(key) == good[-1]
        finally:
            T.mk_set_option(key, old)


def test_decode_refuses_unknown_exec_mode_and_graph_prefill():
    """Argument checks run before anything touches a device: an unknown
    execution mode is refused, and prefill has no graph mode."""
    import ctypes as C
    wl = W.WORKLOADS["layer256_f32"]
    q = T.mk_build_queue(T.make_config(wl.model), T.make_plan(wl.plan, T.MK_DECODE, 1, 129))
    w, kv = L.mk_weights(), L.mk_kv()
    fake = C.c_void_p(0x1000)
    st = L.lib().mk_decode_step(q.handle, fake, C.byref(w), C.byref(kv), None, fake, fake, 1, fake,
                                1 << 30, None, None, 7, None)
    assert st == T.MK_EINVAL
    assert b"null" in L.lib().mk_last_error() or b"exec_mode" in L.lib().mk_last_error()


def test_static_step_refuses_modes_that_allocate():
    """The static-scratch step has neither graph nor multi-stream mode (both
    create runtime objects); the refusal comes before any device call."""
    import ctypes as C
    wl = W.WORKLOADS["layer256_f32"]
    q = T.mk_build_queue(T.make_config(wl.model), T.make_plan(wl.plan, T.MK_DECODE, 1, 129))
    w, kv = L.mk_weights(), L.mk_kv()
    fake = C.c_void_p(0x1000)
    for mode in (T.MK_KERNEL_PER_OP_GRAPH, T.MK_MULTI_STREAM):
        st = L.lib().mk_decode_step_static(q.handle, fake, C.byref(w), C.byref(kv), None, fake, fake, 1, None,
                                           None, None, mode, None)
        assert st == T.MK_EINVAL, mode
        assert b"static-scratch" in L.lib().mk_last_error()


def test_queue_free_accepts_null_and_frees_once():
    L.lib().mk_queue_free(None)
    wl = W.WORKLOADS["layer256_f32"]
    q = T.mk_build_queue(T.make_config(wl.model), T.make_plan(wl.plan, T.MK_DECODE, 1, 129))
    q.close()
    q.close()


@pytest.mark.parametrize("name,rows", [("llama1b_b1", 1), ("llama1b_b1", 3), ("llama8b_b1", 1)])
def test_builder_bytes_loop_queue(name, rows):
    """Loop queues (persistent multi-step decode): LM-head tiles, argmax rows and
    the embedding tiles' previous-step waits agree byte for byte."""
    wl = W.WORKLOADS[name]
    plan = dataclasses.replace(wl.plan, loop=1)
    got, ref = _both(wl.model, plan, QS.MODE_DECODE, rows, wl.run.ctx_max)
    for part in ref:
        assert got[part] == ref[part], part


def test_builder_rejects_loop_without_lm_head():
    wl = W.WORKLOADS["layer256_f32"]
    with pytest.raises(T.MkError):
        T.mk_build_queue(T.make_config(wl.model), T.make_plan(dataclasses.replace(wl.plan, loop=1), T.MK_DECODE,
                                                              1, 129))


@pytest.mark.parametrize("name", ["llama1b_stream_b32", "llama8b_b1"])
def test_builder_bytes_attn_pop(name):
    """Run-time split hand-out: the same instructions, waits and targets as the
    static queue, with bit 3 of the META flags word set; both builders agree."""
    wl = W.WORKLOADS[name]
    plan = dataclasses.replace(wl.plan, attn_pop=1)
    got, ref = _both(wl.model, plan, QS.MODE_DECODE, wl.run.batch, wl.run.ctx_max)
    assert got == ref
    static, _ = _both(wl.model, dataclasses.replace(wl.plan, attn_pop=0), QS.MODE_DECODE, wl.run.batch,
                      wl.run.ctx_max)
    for part in got:
        if part != "meta":
            assert got[part] == static[part], part
    flags = np.frombuffer(got["meta"][:80], dtype="<u4")[19]
    assert flags & 8 and not np.frombuffer(static["meta"][:80], dtype="<u4")[19] & 8


@pytest.mark.parametrize("bad", [dict(attn_pop=2), dict(attn_pop=-1), dict(attn_pop=1, loop=1)])
def test_builder_rejects_bad_attn_pop(bad):
    wl = W.WORKLOADS["llama1b_b1"]
    plan = dataclasses.replace(wl.plan, **bad)
    with pytest.raises(T.MkError):
        T.mk_build_queue(T.make_config(wl.model), T.make_plan(plan, QS.MODE_DECODE, 1, wl.run.ctx_max))
    with pytest.raises(QS.QueueError):
        QS.build(wl.model, plan, QS.MODE_DECODE, 1, wl.run.ctx_max)


def test_prefill_rejects_attn_pop():
    wl = W.WORKLOADS["qwen8b_prefill"]
    plan = dataclasses.replace(wl.plan, attn_pop=1)
    with pytest.raises(T.MkError):
        T.mk_build_queue(T.make_config(wl.model), T.make_plan(plan, QS.MODE_PREFILL, 256, 512))
    with pytest.raises(QS.QueueError):
        QS.build(wl.model, plan, QS.MODE_PREFILL, 256, 512)


def test_workspace_holds_the_split_counters():
    wl = W.WORKLOADS["llama1b_stream_b32"]
    mk = lambda pop: T.mk_build_queue(T.make_config(wl.model),
                                      T.make_plan(dataclasses.replace(wl.plan, attn_pop=pop), T.MK_DECODE,
                                                  wl.run.batch, wl.run.ctx_max))
    q0, q1 = mk(0), mk(1)
    # one 128-byte counter line per layer after the sub-queue heads
    grow = q1.workspace_offset(T.MK_T_ERROR) - q0.workspace_offset(T.MK_T_ERROR)
    assert grow == ((256 + 16) * 128 + 255) // 256 * 256 - (256 * 128 + 255) // 256 * 256
