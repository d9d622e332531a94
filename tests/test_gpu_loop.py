"""Persistent multi-step decode (mk_decode_loop) on the GPU.

One launch runs T decode steps of a loop queue: each step's LM-head tiles and
argmax run inside the megakernel, and the next step's embedding tiles wait on
the previous step's argmax.  Checked against the float64 oracle step by step
(teacher-forced ids), against T single-step launches of the same op bodies
(the last step's hidden rows bit for bit), for greedy feedback (the chain of
argmaxes equals a teacher-forced run fed with that chain), and under a
NaN-poisoned workspace with seeded producer delays.  Tolerance 2e-2 per row
(bf16 model).
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
STEPS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(batch, ctx0, n_queues, loop=1):
    from _gpucase import make_case
    base = W.shrink(W.WORKLOADS["llama1b_b1"], n_layers=2, vocab=4096, batch=batch, ctx0=ctx0, steps=STEPS,
                    name=f"llama1b_L2_V4096_B{batch}_loop{loop}")
    wl = dataclasses.replace(base, plan=W.Plan(tf=32, td=8, n_queues=n_queues, loop=loop))
    return make_case(wl, gain_jitter=0.1)


def _run_loop(c, tokens, feedback, steps=STEPS):
    """One mk_decode_loop call from the initial cache: (logits [T,B,V], next [T,B], X_L of the last step)."""
    B, V = c.wl.run.batch, c.m.vocab
    c.reset_kv()
    ctx = torch.tensor(c.wl.run.ctx0, dtype=torch.int32, device="cuda")
    tok = torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)).cuda()
    lg = torch.full((steps, B, V), float("nan"), dtype=torch.float32, device="cuda")
    nx = torch.full((steps, B), -1, dtype=torch.int32, device="cuda")
    T.mk_decode_loop(c.q, c.dq, c.dm.w, c.dkv.kv, tok, ctx, B, steps, feedback, c.ws, lg, nx)
    torch.cuda.synchronize()
    err = T.mk_device_error(c.q, c.ws)
    assert err.code == 0, (err.code, err.instr, err.barrier, err.value, err.target)
    tg = np.frombuffer(c.q.export(T.MK_PART_TARGETS), dtype=np.uint32).astype(np.int64)
    assert np.array_equal(c.counters().astype(np.int64), tg * steps), "counters must end at steps x targets"
    return lg.cpu().numpy(), nx.cpu().numpy(), c.tensor(T.MK_T_X, c.m.n_layers, c.m.hidden)


@pytest.mark.parametrize("batch,ctx0,nq", [(1, (1024,), 256), (3, (900, 31, 511), 8),
                                           (20, tuple(900 - 41 * b for b in range(20)), 256)],
                         ids=["b1_static", "b3_shared8", "b20_static"])
def test_loop_teacher_forced_matches_oracle(batch, ctx0, nq):
    from _gpucase import log
    c = _case(batch, ctx0, nq)
    lg, nx, xl = _run_loop(c, c.tokens[:STEPS], feedback=0)
    model = c.oracle_model()
    K, V = c.K0.copy(), c.V0.copy()
    errs = {}
    for t in range(STEPS):
        tr = N.decode_step(model, K, V, [p + t for p in ctx0], tokens=c.tokens[t])
        errs[f"logits{t}"] = N.max_rel_err_rows(lg[t].astype(np.float64), tr.logits)
        assert np.array_equal(nx[t], N.argmax_lowest(lg[t])), t
    errs["x_out"] = N.max_rel_err_rows(xl, tr.x_out)
    Kg, Vg = c.kv_host()
    for t in range(STEPS):
        for b, p in enumerate(ctx0):
            errs[f"k{t}"] = max(errs.get(f"k{t}", 0.0), N.max_rel_err(N.to_f64(Kg[:, b, :, p + t]),
                                                                      N.to_f64(K[:, b, :, p + t])))
    worst = max(errs, key=errs.get)
    log(f"    loop B={batch} n_queues={nq}: worst {worst} = {errs[worst]:.3e}")
    assert errs[worst] <= TOL, errs


def test_loop_last_hidden_rows_equal_single_steps():
    """The layers of each step run the same op bodies on the same tiles as
    mk_decode_step: after T steps the hidden rows and the cache are
    bit-identical to T single-step launches; the in-kernel LM head (the GEMV
    body) agrees with the separate LM-head kernel to rounding."""
    ncu = T.mk_get_option(T.MK_OPT_NUM_CUS)
    ctx0 = (700, 1100)
    cl = _case(2, ctx0, ncu, loop=1)
    lg, nx, xl = _run_loop(cl, cl.tokens[:STEPS], feedback=0)
    k_loop = cl.kv_host()[0].copy()
    cs = _case(2, ctx0, ncu, loop=0)
    cs.reset_kv()
    for t in range(STEPS):
        cs.step(t, [p + t for p in ctx0], T.MK_MEGAKERNEL)
        assert N.max_rel_err_rows(lg[t].astype(np.float64), cs.logits.cpu().numpy().astype(np.float64)) < 1e-5
    assert np.array_equal(xl, cs.tensor(T.MK_T_X, cs.m.n_layers, cs.m.hidden))
    assert np.array_equal(k_loop, cs.kv_host()[0])


def test_loop_greedy_feedback_chain():
    """feedback = 1: step t + 1 embeds step t's argmax, and the run equals the
    teacher-forced run fed with that chain of ids, bit for bit."""
    from _gpucase import log
    c = _case(2, (1000, 333), 256)
    lg_g, nx_g, xl_g = _run_loop(c, c.tokens[0], feedback=1)
    for t in range(STEPS):
        assert np.array_equal(nx_g[t], N.argmax_lowest(lg_g[t])), t
    chain = np.stack([c.tokens[0]] + [nx_g[t] for t in range(STEPS - 1)])
    lg_t, nx_t, xl_t = _run_loop(c, chain, feedback=0)
    assert np.array_equal(lg_g, lg_t) and np.array_equal(nx_g, nx_t) and np.array_equal(xl_g, xl_t)
    log(f"    greedy chain {chain[:, 0].tolist()} -> {nx_g[-1].tolist()}")


def test_loop_poisoned_and_delayed_runs_are_bit_identical():
    c = _case(2, (1000, 333), 8)
    clean = _run_loop(c, c.tokens[:STEPS], feedback=0)
    for seed in (1, 2):
        c.ws.fill_(255)
        T.mk_set_option(T.MK_OPT_DELAY_SEED, seed)
        try:
            got = _run_loop(c, c.tokens[:STEPS], feedback=0)
        finally:
            T.mk_set_option(T.MK_OPT_DELAY_SEED, 0)
        for a, b in zip(clean, got):
            assert np.array_equal(a, b), seed


def test_loop_refuses_wrong_queues_and_arguments():
    c = _case(1, (100,), 256, loop=0)
    tok = torch.zeros((STEPS, 1), dtype=torch.int32, device="cuda")
    ctx = torch.tensor([100], dtype=torch.int32, device="cuda")
    nx = torch.zeros((STEPS, 1), dtype=torch.int32, device="cuda")
    with pytest.raises(T.MkError) as ei:
        T.mk_decode_loop(c.q, c.dq, c.dm.w, c.dkv.kv, tok, ctx, 1, STEPS, 0, c.ws, None, nx)
    assert ei.value.status == T.MK_EINVAL
    cl = _case(1, (100,), 256, loop=1)
    for steps, fb in ((0, 0), (2, 3)):
        with pytest.raises(T.MkError):
            T.mk_decode_loop(cl.q, cl.dq, cl.dm.w, cl.dkv.kv, tok, ctx, 1, steps, fb, cl.ws, None, nx)
    with pytest.raises(T.MkError):
        T.mk_decode_step(cl.q, cl.dq, cl.dm.w, cl.dkv.kv, tok[0], None, ctx, 1, cl.ws, None, None,
                         T.MK_MEGAKERNEL)
