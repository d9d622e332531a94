"""Compositions of several megakernels per decode step (MK_OPT_MEGAKERNELS).

With K > 1 the step is K megakernel launches on one stream, cut at layer
boundaries: launch k runs the queue positions of layers [k L / K, (k+1) L / K)
(the first also the embedding).  Each launch runs the same op bodies over the
same tile schedule; waits on tiles of an earlier launch are met because that
launch has finished.  Every output (each layer's intermediates, the new cache
entries, logits, argmax) must therefore equal the single megakernel's bit for
bit, with the split partials merged by COMBINE tiles or in the last split,
with splits handed out at run time, and also with a NaN-poisoned workspace and
seeded producer delays.  Plans with shared sub-queues and more launches than
layers are refused before anything is launched.
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
    T.mk_set_option(T.MK_OPT_MEGAKERNELS, 1)
    T.mk_set_option(T.MK_OPT_DELAY_SEED, 0)


def _cases():
    ncu = 256
    b1 = W.shrink(W.WORKLOADS["llama1b_b1"], n_layers=4, vocab=4096, batch=1, ctx0=(1024,), steps=1,
                  name="llama1b_L4_B1")
    b4 = W.shrink(W.WORKLOADS["llama1b_stream_b32"], n_layers=4, vocab=4096, batch=4,
                  ctx0=(3000, 37, 600, 1), steps=1, name="llama1b_L4_B4")
    b4 = dataclasses.replace(b4, plan=dataclasses.replace(b4.plan, kb=512))     # several splits per row
    e8 = W.shrink(W.WORKLOADS["llama8b_b1"], n_layers=3, vocab=4096, steps=1, name="llama8b_L3_B1")
    return {
        "bf16_1b_b1_combine": dataclasses.replace(b1, plan=W.Plan(tf=32, td=8, n_queues=ncu)),
        "bf16_1b_b1_merge_last": b1,
        "bf16_1b_b4_split_popped": b4,
        "bf16_8b_b1_merge_last": e8,
    }


def _outputs(c):
    m = c.m
    out = {f"x{l}": c.tensor(T.MK_T_X, l, m.hidden) for l in range(m.n_layers + 1)}
    for l in range(m.n_layers):
        out[f"qkv{l}"] = c.tensor(T.MK_T_QKV, l, m.qkv_cols)
        out[f"att{l}"] = c.tensor(T.MK_T_ATT, l, m.attn_cols)
        out[f"h{l}"] = c.tensor(T.MK_T_HRES, l, m.hidden)
        out[f"act{l}"] = c.tensor(T.MK_T_ACT, l, m.ffn)
    out["logits"] = c.logits.cpu().numpy().copy()
    out["next"] = c.nxt.cpu().numpy().copy()
    k, v = c.kv_host()
    out["k"], out["v"] = k.copy(), v.copy()
    return out


def _run(c, launches, poison=False, seed=0):
    c.reset_kv()
    if poison:
        c.ws.fill_(255)
        c.logits.fill_(float("nan"))
        c.nxt.fill_(-1)
    T.mk_set_option(T.MK_OPT_MEGAKERNELS, launches)
    T.mk_set_option(T.MK_OPT_DELAY_SEED, seed)
    try:
        c.step(0, list(c.wl.run.ctx0), T.MK_MEGAKERNEL)
    finally:
        T.mk_set_option(T.MK_OPT_DELAY_SEED, 0)
        T.mk_set_option(T.MK_OPT_MEGAKERNELS, 1)
    err = T.mk_device_error(c.q, c.ws)
    assert err.code == 0, (err.code, err.instr, err.barrier, err.value, err.target)
    tg = np.frombuffer(c.q.export(T.MK_PART_TARGETS), dtype=np.uint32)
    assert np.array_equal(c.counters(), tg), "counters must end at their targets"
    return _outputs(c)


def _diff(a, b):
    return [k for k in a if not np.array_equal(a[k], b[k])]


@pytest.mark.parametrize("name", list(_cases()))
def test_composition_equals_one_megakernel_bitwise(name):
    from _gpucase import make_case, log
    c = make_case(_cases()[name], gain_jitter=0.1)
    ref = _run(c, 1)
    for k, v in ref.items():
        if v.dtype.kind == "f":
            assert np.isfinite(v).all(), k
    for launches in range(2, c.m.n_layers + 1):
        bad = _diff(ref, _run(c, launches))
        log(f"    {name} launches={launches}: {'identical' if not bad else 'DIFFERS in ' + ','.join(bad[:6])}")
        assert not bad, (launches, bad)


@pytest.mark.parametrize("name", ["bf16_1b_b1_merge_last", "bf16_1b_b4_split_popped"])
def test_composition_poisoned_and_delayed_runs_are_bit_identical(name):
    from _gpucase import make_case, log
    c = make_case(_cases()[name], gain_jitter=0.1)
    clean = _run(c, 3)
    for seed in (1, 2):
        bad = _diff(clean, _run(c, 3, poison=True, seed=seed))
        log(f"    {name} seed {seed}: {'identical' if not bad else 'DIFFERS in ' + ','.join(bad[:6])}")
        assert not bad, (seed, bad)


def test_composition_refusals():
    """More launches than layers, and a plan whose workers share sub-queues,
    are refused with MK_ENOTSUP; the next plain step still runs."""
    from _gpucase import make_case
    cases = _cases()
    c = make_case(cases["bf16_1b_b1_merge_last"])
    T.mk_set_option(T.MK_OPT_MEGAKERNELS, c.m.n_layers + 1)
    with pytest.raises(T.MkError) as e:
        c.step(0, list(c.wl.run.ctx0), T.MK_MEGAKERNEL)
    assert e.value.status == T.MK_ENOTSUP
    shared = dataclasses.replace(cases["bf16_1b_b1_combine"], plan=W.Plan(n_queues=8))
    s = make_case(shared)
    T.mk_set_option(T.MK_OPT_MEGAKERNELS, 2)
    with pytest.raises(T.MkError) as e:
        s.step(0, list(s.wl.run.ctx0), T.MK_MEGAKERNEL)
    assert e.value.status == T.MK_ENOTSUP
    T.mk_set_option(T.MK_OPT_MEGAKERNELS, 1)
    _run(c, 1)


def test_composition_through_the_static_scratch_entry():
    """mk_decode_step_static runs the same compositions: with two launches per
    step its logits, argmax and new cache entries equal one launch on a
    caller-allocated workspace, bit for bit."""
    from _gpucase import make_case
    c = make_case(_cases()["bf16_1b_b1_merge_last"], gain_jitter=0.1)
    assert c.q.workspace_nbytes() <= T.MK_STATIC_SCRATCH_BYTES
    ref = _run(c, 1)
    B = c.wl.run.batch
    c.reset_kv()
    lg = torch.full_like(c.logits, float("nan"))
    nx = torch.full_like(c.nxt, -1)
    err = torch.full((8,), 0xFFFF, dtype=torch.int32, device="cuda")
    tok = torch.from_numpy(c.tokens[0].astype(np.int32)).cuda()
    cl = torch.tensor(list(c.wl.run.ctx0), dtype=torch.int32, device="cuda")
    T.mk_set_option(T.MK_OPT_MEGAKERNELS, 2)
    try:
        T.mk_decode_step_static(c.q, c.dq, c.dm.w, c.dkv.kv, tok, None, cl, B, lg, nx, err, T.MK_MEGAKERNEL)
        torch.cuda.synchronize()
    finally:
        T.mk_set_option(T.MK_OPT_MEGAKERNELS, 1)
    assert (err.cpu().numpy() == 0).all()
    k, v = c.kv_host()
    assert np.array_equal(lg.cpu().numpy(), ref["logits"])
    assert np.array_equal(nx.cpu().numpy(), ref["next"])
    assert np.array_equal(k, ref["k"]) and np.array_equal(v, ref["v"])
