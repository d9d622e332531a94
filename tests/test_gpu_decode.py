"""GPU parity of the decode path through the C ABI against the float64 oracle.

Tolerances (max |gpu - oracle| / max |oracle| per tensor, step and row): 1e-4
for the fp32 model, 2e-2 for the bf16 models.  Megakernel and kernel-per-op
modes run the same op bodies and must agree bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import tile_synchronized_decoder_amd as T
import workloads as W
from oracle import numerics as N
from oracle import queue_spec as QS

pytestmark = pytest.mark.gpu

TOL_F32, TOL_BF16 = 1e-4, 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from _gpucase import log
    log(f"[gpu] {torch.cuda.get_device_name(0)} lib={T.library_path()}")


def rel_rows(got, ref):
    return max(N.max_rel_err(got[b], ref[b]) for b in range(ref.shape[0]))


def check_step(c, tr, tol, layers=None):
    """Compare workspace intermediates of one step with an oracle trace.  A
    queue with fused split combines writes no attention-output tensor (the
    O-projection merges the partials itself); its error shows in HRES."""
    m = c.m
    errs = {}
    fused = getattr(c.wl.plan, "fuse_combine", 0)
    for l in (layers if layers is not None else range(m.n_layers)):
        if not fused:
            errs[f"att{l}"] = rel_rows(c.tensor(T.MK_T_ATT, l, m.attn_cols), tr.attn[l])
        errs[f"h{l}"] = rel_rows(c.tensor(T.MK_T_HRES, l, m.hidden), tr.h[l])
        errs[f"act{l}"] = rel_rows(c.tensor(T.MK_T_ACT, l, m.ffn), tr.act[l])
        hres = c.tensor(T.MK_T_HRES, l, m.hidden)
        xin = c.tensor(T.MK_T_X, l, m.hidden)
        xout = c.tensor(T.MK_T_X, l + 1, m.hidden)
        errs[f"attn_branch{l}"] = rel_rows(hres - xin, tr.attn_branch[l])
        errs[f"mlp_branch{l}"] = rel_rows(xout - hres, tr.mlp_branch[l])
    errs["x_out"] = rel_rows(c.tensor(T.MK_T_X, m.n_layers, m.hidden), tr.x_out)
    if c.logits is not None:
        lg = c.logits.cpu().numpy().astype(np.float64)
        errs["logits"] = rel_rows(lg, tr.logits)
        nx = c.nxt.cpu().numpy()
        assert np.array_equal(nx, N.argmax_lowest(c.logits.cpu().numpy())), "argmax of the GPU logits"
    worst = max(errs, key=errs.get)
    from _gpucase import log
    log(f"    worst {worst} = {errs[worst]:.3e}")
    assert errs[worst] <= tol, errs
    return errs


# ----------------------------------------------------------------------------- single fp32 layer

@pytest.fixture(scope="module")
def small():
    from _gpucase import make_case
    return make_case(W.WORKLOADS["layer256_f32"], gain_jitter=0.1)


@pytest.mark.parametrize("mode", [T.MK_MEGAKERNEL, T.MK_KERNEL_PER_OP], ids=["mega", "kpo"])
def test_layer_fp32_matches_oracle(small, mode):
    c = small
    c.reset_kv()
    c.step(0, [128], mode)
    K, V = c.K0.copy(), c.V0.copy()
    tr = N.decode_step(c.oracle_model(), K, V, [128], x0=c.x0[0])
    check_step(c, tr, TOL_F32)
    Kg, Vg = c.kv_host()
    assert N.max_rel_err(Kg[0, 0, :, 128], K[0, 0, :, 128]) < TOL_F32
    assert N.max_rel_err(Vg[0, 0, :, 128], V[0, 0, :, 128]) < TOL_F32
    # only position 128 changed
    assert np.array_equal(Kg[0, 0, :, :128], c.K0[0, 0, :, :128])


def test_layer_modes_bitwise_equal_and_counters(small):
    c = small
    outs = {}
    for mode in (T.MK_KERNEL_PER_OP, T.MK_MEGAKERNEL, T.MK_MEGAKERNEL):
        c.reset_kv()
        c.ws.zero_()
        c.step(0, [128], mode)
        snap = {k: c.tensor(kind, 0, cols) for k, kind, cols in
                (("att", T.MK_T_ATT, 256), ("h", T.MK_T_HRES, 256), ("act", T.MK_T_ACT, 688),
                 ("x", T.MK_T_X, 256))}
        snap["x"] = c.tensor(T.MK_T_X, 1, 256)
        Kg, Vg = c.kv_host()
        snap["k"], snap["v"] = Kg, Vg
        if mode == T.MK_MEGAKERNEL:
            tg = np.frombuffer(c.q.export(T.MK_PART_TARGETS), dtype=np.uint32)
            assert np.array_equal(c.counters(), tg), "counters must equal targets after the step"
            err = T.mk_device_error(c.q, c.ws)
            assert err.code == 0
        outs.setdefault(mode, []).append(snap)
    a, b, b2 = outs[T.MK_KERNEL_PER_OP][0], outs[T.MK_MEGAKERNEL][0], outs[T.MK_MEGAKERNEL][1]
    for k in a:
        assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(b[k], b2[k]), k


@pytest.mark.parametrize("ctx", [0, 1, 31, 32, 64, 127])
def test_layer_fp32_short_contexts(small, ctx):
    c = small
    c.reset_kv()
    c.step(0, [ctx], T.MK_MEGAKERNEL)
    tr = N.decode_step(c.oracle_model(), c.K0.copy(), c.V0.copy(), [ctx], x0=c.x0[0])
    check_step(c, tr, TOL_F32)


def test_layer_fp32_batch_ragged_tiles_subqueues():
    from _gpucase import make_case
    wl = W.WORKLOADS["layer256_f32"]
    wl = W.Workload("layer256_b3_ragged", wl.model,
                    W.RunConfig(batch=3, ctx0=(5, 128, 64), steps=1, ctx_max=129, seed=9),
                    W.Plan(tq=24, to=40, tf=56, td=24, kb=48, n_queues=8))
    c = make_case(wl, gain_jitter=0.1)
    tr = N.decode_step(c.oracle_model(), c.K0.copy(), c.V0.copy(), list(wl.run.ctx0), x0=c.x0[0])
    for mode in (T.MK_MEGAKERNEL, T.MK_KERNEL_PER_OP):
        c.reset_kv()
        c.step(0, list(wl.run.ctx0), mode)
        check_step(c, tr, TOL_F32)


# ----------------------------------------------------------------------------- bf16, 1B-shaped

def _shrunk_1b(layers=2, vocab=4096, batch=1, ctx0=(1024,), steps=3):
    base = W.WORKLOADS["llama1b_b1"]
    wl = W.shrink(base, n_layers=layers, vocab=vocab, batch=batch, ctx0=ctx0, steps=steps,
                  name=f"llama1b_L{layers}_V{vocab}_B{batch}")
    return dataclasses.replace(wl, plan=W.Plan())         # one shared sub-queue, default tiles


# 5 and 20 rows fill their row buckets (8 and 32) only partly: the matrix-core
# GEMV's staging and B columns past the batch
@pytest.mark.parametrize("batch", [1, 4, 5, 20, 32])
def test_bf16_shrunk_multistep_matches_oracle(batch):
    from _gpucase import make_case, log
    ctx0 = tuple(1024 - 29 * b for b in range(batch))
    wl = _shrunk_1b(batch=batch, ctx0=ctx0)
    c = make_case(wl)
    model = c.oracle_model()
    K, V = c.K0.copy(), c.V0.copy()
    for t in range(wl.run.steps):
        ctx = [p + t for p in ctx0]
        tr = N.decode_step(model, K, V, ctx, tokens=c.tokens[t])
        c.step(t, ctx, T.MK_MEGAKERNEL)
        log(f"  step {t}")
        check_step(c, tr, TOL_BF16)
    Kg, _ = c.kv_host()
    # the cache rows written by the steps agree with the oracle's (bf16, rounding may differ by an ulp)
    for t in range(wl.run.steps):
        for b in range(batch):
            p = ctx0[b] + t
            assert N.max_rel_err(N.to_f64(Kg[:, b, :, p]), N.to_f64(K[:, b, :, p])) < 1e-2


@pytest.mark.parametrize("ctx0", [(700, 1100), (700, 1100, 33, 512, 1023, 64)], ids=["b2", "b6"])
def test_bf16_shrunk_modes_bitwise_equal(ctx0):
    from _gpucase import make_case
    wl = _shrunk_1b(batch=len(ctx0), ctx0=ctx0, steps=1)
    c = make_case(wl)
    res = []
    for mode in (T.MK_MEGAKERNEL, T.MK_KERNEL_PER_OP, T.MK_MEGAKERNEL):
        c.reset_kv()
        c.step(0, list(ctx0), mode)
        res.append((c.logits.cpu().numpy().copy(), c.tensor(T.MK_T_X, 2, 2048), c.kv_host()[0]))
    for r in res[1:]:
        for a, b in zip(res[0], r):
            assert np.array_equal(a, b)


def test_bf16_one_subqueue_per_worker():
    """With as many sub-queues as workers every worker runs a fixed list of
    instructions (no pops, records loaded one ahead); results match the oracle
    and the kernel-per-op mode bit for bit, also with 256-tile GEMV ops."""
    from _gpucase import make_case, log
    ncu = T.mk_get_option(T.MK_OPT_NUM_CUS)
    base = _shrunk_1b(batch=2, ctx0=(700, 1100), steps=2)
    for tiles in (dict(), dict(tq=12, to=8, tf=32, td=8, kb=128)):
        wl = dataclasses.replace(base, plan=dataclasses.replace(base.plan, n_queues=ncu, **tiles))
        c = make_case(wl)
        model = c.oracle_model()
        K, V = c.K0.copy(), c.V0.copy()
        for t in range(wl.run.steps):
            ctx = [700 + t, 1100 + t]
            tr = N.decode_step(model, K, V, ctx, tokens=c.tokens[t])
            c.step(t, ctx, T.MK_MEGAKERNEL)
            log(f"  tiles {tiles} step {t}")
            check_step(c, tr, TOL_BF16)
            mega = (c.logits.cpu().numpy().copy(), c.tensor(T.MK_T_X, 2, 2048))
            c.step(t, ctx, T.MK_KERNEL_PER_OP)
            assert np.array_equal(c.logits.cpu().numpy(), mega[0])
            assert np.array_equal(c.tensor(T.MK_T_X, 2, 2048), mega[1])


def test_bf16_separate_lm_head_matches_fused():
    """mk_decode_step without outputs followed by mk_lm_head gives the logits
    and argmax of mk_decode_step with outputs, bit for bit, in both modes."""
    from _gpucase import make_case
    wl = _shrunk_1b(batch=2, ctx0=(700, 1100), steps=1)
    c = make_case(wl)
    m, B = c.m, 2
    tok = torch.from_numpy(c.tokens[0].astype(np.int32)).cuda()
    cl = torch.tensor([700, 1100], dtype=torch.int32, device="cuda")
    for mode in (T.MK_MEGAKERNEL, T.MK_KERNEL_PER_OP):
        c.reset_kv()
        c.step(0, [700, 1100], mode)
        fused = (c.logits.cpu().numpy().copy(), c.nxt.cpu().numpy().copy())
        c.reset_kv()
        lg = torch.full((B, m.vocab), -1.0, dtype=torch.float32, device="cuda")
        nx = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        T.mk_decode_step(c.q, c.dq, c.dm.w, c.dkv.kv, tok, None, cl, B, c.ws, None, None, mode)
        T.mk_lm_head(c.q, c.dm.w, c.ws, lg, nx)
        torch.cuda.synchronize()
        assert np.array_equal(lg.cpu().numpy(), fused[0])
        assert np.array_equal(nx.cpu().numpy(), fused[1])


# ----------------------------------------------------------------------------- full Llama-3-1B shape

@pytest.mark.slow
def test_llama1b_full_size_steps():
    """The full 16-layer, 128256-vocab model: the first steps of the timed workload."""
    from _gpucase import make_case, log
    wl = W.shrink(W.WORKLOADS["llama1b_b1"], steps=3)
    c = make_case(wl)
    model = c.oracle_model()
    K, V = c.K0.copy(), c.V0.copy()
    for t in range(wl.run.steps):
        ctx = [1024 + t]
        tr = N.decode_step(model, K, V, ctx, tokens=c.tokens[t])
        for mode in (T.MK_KERNEL_PER_OP, T.MK_MEGAKERNEL):
            c.step(t, ctx, mode)
            log(f"  step {t} mode {mode}")
            check_step(c, tr, TOL_BF16, layers=[0, 7, 15])


# ----------------------------------------------------------------------------- failure handling

def test_watchdog_reports_unreachable_barrier(small):
    """A queue whose first barrier target can never be reached: the bounded
    waits expire, the kernel drains, and the error record names the wait."""
    c = small
    parts = c.q.export(T.MK_PART_DEVICE)
    img = np.frombuffer(parts, dtype=np.uint8).copy()
    tg_off = (c.q.nbytes(T.MK_PART_INSTR) + 255) // 256 * 256
    tg_off += (c.q.nbytes(T.MK_PART_WAITS) + 255) // 256 * 256
    targets = img[tg_off: tg_off + c.q.nbytes(T.MK_PART_TARGETS)].view(np.uint32)
    targets[0] += 1                          # QKV tile 0 signals once; nobody reaches 2
    bad = torch.from_numpy(img).cuda()
    old = T.mk_get_option(T.MK_OPT_SPIN_LIMIT)
    T.mk_set_option(T.MK_OPT_SPIN_LIMIT, 20000)
    try:
        c.reset_kv()
        cl = torch.tensor([128], dtype=torch.int32, device="cuda")
        x0 = torch.from_numpy(c.x0[0]).cuda()
        T.mk_decode_step(c.q, bad, c.dm.w, c.dkv.kv, None, x0, cl, 1, c.ws, None, None, T.MK_MEGAKERNEL)
        err = T.mk_device_error(c.q, c.ws)
    finally:
        T.mk_set_option(T.MK_OPT_SPIN_LIMIT, old)
    assert err.code == 1 and err.value < err.target
    # the next good step clears the record and is correct again
    c.reset_kv()
    c.step(0, [128], T.MK_MEGAKERNEL)
    assert T.mk_device_error(c.q, c.ws).code == 0


def test_workers_that_cannot_all_be_resident_are_refused(small):
    """A persistent interpreter needs every workgroup resident at once (workers
    wait on each other's tiles).  Eight workgroups per compute unit do not fit
    the interpreter's shared memory: the launch is refused up front, nothing
    runs, and the default launch works again afterwards."""
    c = small
    old = T.mk_get_option(T.MK_OPT_WORKERS_PER_CU)
    T.mk_set_option(T.MK_OPT_WORKERS_PER_CU, 8)
    try:
        c.reset_kv()
        with pytest.raises(T.MkError) as ei:
            c.step(0, [128], T.MK_MEGAKERNEL)
        assert ei.value.status == T.MK_ENOTSUP
    finally:
        T.mk_set_option(T.MK_OPT_WORKERS_PER_CU, old)
    c.reset_kv()
    c.step(0, [128], T.MK_MEGAKERNEL)
    assert T.mk_device_error(c.q, c.ws).code == 0


# ----------------------------------------------------------------------------- fused split combines

def _fused(wl, **kw):
    return dataclasses.replace(wl, plan=dataclasses.replace(wl.plan, fuse_combine=1, **kw))


@pytest.mark.parametrize("ctx", [0, 31, 128])
def test_fused_combine_fp32_layer_both_modes(ctx):
    """Split combines fused into the O-projection: oracle parity on the fp32
    layer (5 splits, empty ones at short contexts), megakernel and per-op bit
    for bit, counters equal to targets."""
    from _gpucase import make_case
    c = make_case(_fused(W.WORKLOADS["layer256_f32"]), gain_jitter=0.1)
    outs = []
    for mode in (T.MK_MEGAKERNEL, T.MK_KERNEL_PER_OP):
        c.reset_kv()
        c.ws.zero_()
        c.step(0, [ctx], mode)
        tr = N.decode_step(c.oracle_model(), c.K0.copy(), c.V0.copy(), [ctx], x0=c.x0[0])
        check_step(c, tr, TOL_F32)
        outs.append((c.tensor(T.MK_T_HRES, 0, 256), c.tensor(T.MK_T_X, 1, 256)))
        if mode == T.MK_MEGAKERNEL:
            tg = np.frombuffer(c.q.export(T.MK_PART_TARGETS), dtype=np.uint32)
            assert np.array_equal(c.counters(), tg)
            assert T.mk_device_error(c.q, c.ws).code == 0
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("ctx0", [(1024,), (100,)])
def test_fused_combine_bf16_multistep(ctx0):
    """The 1B shape at batch 1 (five 256-key splits, all but one empty at
    context 100): three steps against the oracle, megakernel = per-op."""
    from _gpucase import make_case, log
    wl = _fused(_shrunk_1b(batch=1, ctx0=ctx0))
    c = make_case(wl)
    model = c.oracle_model()
    K, V = c.K0.copy(), c.V0.copy()
    for t in range(wl.run.steps):
        ctx = [p + t for p in ctx0]
        tr = N.decode_step(model, K, V, ctx, tokens=c.tokens[t])
        c.step(t, ctx, T.MK_MEGAKERNEL)
        log(f"  fused step {t}")
        check_step(c, tr, TOL_BF16)
        mega = (c.logits.cpu().numpy().copy(), c.tensor(T.MK_T_X, wl.model.n_layers, 2048))
        c.step(t, ctx, T.MK_KERNEL_PER_OP)
        assert np.array_equal(c.logits.cpu().numpy(), mega[0])
        assert np.array_equal(c.tensor(T.MK_T_X, wl.model.n_layers, 2048), mega[1])


def test_fused_combine_refused_when_partials_do_not_fit():
    """Many splits (8-key splits of an 8448-position cache): the O-projection
    cannot stage every partial in shared memory, so the step is refused before
    anything runs."""
    from _gpucase import make_case
    wl = _fused(W.WORKLOADS["layer256_f32"], kb=8)
    wl = dataclasses.replace(wl, run=dataclasses.replace(wl.run, ctx_max=8448))
    c = make_case(wl)
    with pytest.raises(T.MkError) as ei:
        c.step(0, [128], T.MK_MEGAKERNEL)
    assert ei.value.status == T.MK_ENOTSUP


# ----------------------------------------------------------------------------- kernel-per-op HIP graph

def test_kpo_graph_replays_match_eager_and_megakernel():
    """MK_KERNEL_PER_OP_GRAPH captures the per-op launches once and replays
    them.  Three steps with new token ids and context lengths written into the
    same device buffers between replays (and the outputs overwritten with NaN),
    twice over: every replay equals the eager per-op step and the megakernel
    bit for bit, cache included."""
    from _gpucase import make_case, log
    wl = _shrunk_1b(batch=2, ctx0=(700, 1100), steps=3)
    c = make_case(wl)
    B = 2
    tok = torch.zeros(B, dtype=torch.int32, device="cuda")
    cl = torch.zeros(B, dtype=torch.int32, device="cuda")

    def run(mode):
        outs = []
        c.reset_kv()
        for t in range(3):
            tok.copy_(torch.from_numpy(c.tokens[t].astype(np.int32)))
            cl.copy_(torch.tensor([700 + t, 1100 + t], dtype=torch.int32))
            c.logits.fill_(float("nan"))
            c.nxt.fill_(-1)
            torch.cuda.synchronize()
            T.mk_decode_step(c.q, c.dq, c.dm.w, c.dkv.kv, tok, None, cl, B, c.ws, c.logits, c.nxt, mode)
            torch.cuda.synchronize()
            assert T.mk_device_error(c.q, c.ws).code == 0
            outs.append((c.logits.cpu().numpy().copy(), c.nxt.cpu().numpy().copy(),
                         c.tensor(T.MK_T_X, 2, 2048), c.tensor(T.MK_T_ACT, 1, 8192)))
        outs.append((c.kv_host()[0].copy(), c.kv_host()[1].copy()))
        return outs

    eager = run(T.MK_KERNEL_PER_OP)
    for name, mode in (("graph", T.MK_KERNEL_PER_OP_GRAPH), ("graph replay", T.MK_KERNEL_PER_OP_GRAPH),
                       ("megakernel", T.MK_MEGAKERNEL)):
        got = run(mode)
        for t, (a, b) in enumerate(zip(eager, got)):
            for x, y in zip(a, b):
                assert np.array_equal(x, y), (name, t)
        log(f"    {name}: bit-identical to eager per-op over 3 steps")
    # a new workspace is a new set of arguments: captured again, same results
    c.ws = torch.zeros_like(c.ws)
    again = run(T.MK_KERNEL_PER_OP_GRAPH)
    assert all(np.array_equal(x, y) for a, b in zip(eager, again) for x, y in zip(a, b))


@pytest.mark.parametrize("fuse", [0, 2])
def test_attn_pop_matches_static_order_and_oracle(fuse):
    """Attention splits handed out at run time (plan attn_pop): with ragged
    contexts over 128-key splits the megakernel's results equal the static
    order's and the per-op kernels' bit for bit, and the oracle's."""
    from _gpucase import make_case, log
    ctx0 = (1024, 37, 600, 1, 300, 900)
    wl = W.shrink(W.WORKLOADS["llama1b_b1"], n_layers=2, vocab=4096, batch=len(ctx0), ctx0=ctx0, steps=1,
                  name="llama1b_L2_B6_pop")
    plans = {pop: W.Plan(tf=32, td=8, kb=128, n_queues=256, fuse_combine=fuse, attn_pop=pop) for pop in (0, 1)}
    res = {}
    for pop, plan in plans.items():
        c = make_case(dataclasses.replace(wl, plan=plan))
        for mode in (T.MK_MEGAKERNEL, T.MK_KERNEL_PER_OP):
            c.reset_kv()
            c.step(0, list(ctx0), mode)
            err = T.mk_device_error(c.q, c.ws)
            assert err.code == 0, (err.code, err.instr)
            res[(pop, mode)] = (c.logits.cpu().numpy().copy(), c.tensor(T.MK_T_X, 2, 2048), c.kv_host()[0].copy())
        if pop:
            model = c.oracle_model()
            tr = N.decode_step(model, c.K0.copy(), c.V0.copy(), list(ctx0), tokens=c.tokens[0])
            c.reset_kv()
            c.step(0, list(ctx0), T.MK_MEGAKERNEL)
            check_step(c, tr, TOL_BF16)
    ref = res[(0, T.MK_MEGAKERNEL)]
    for key, got in res.items():
        for a, b in zip(ref, got):
            assert np.array_equal(a, b), key
    log(f"    attn_pop, fuse {fuse}: megakernel and per-op, static and run-time hand-out identical")
