"""mk_decode_step_static: the decode step on the library's static device scratch,
for callers that cannot allocate.  Its outputs equal mk_decode_step's with a
caller-allocated workspace, bit for bit, on two calls in a row, the second
with a smaller input (the scratch keeps the first call's contents); a queue
whose workspace exceeds the scratch is refused before anything runs."""
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


def _case(batch, ctx0, n_queues):
    from _gpucase import make_case
    wl = W.shrink(W.WORKLOADS["llama1b_b1"], n_layers=2, vocab=4096, batch=batch, ctx0=ctx0, steps=2,
                  name=f"llama1b_L2_B{batch}")
    wl = dataclasses.replace(wl, plan=W.Plan(tf=32, td=8, n_queues=n_queues))
    return make_case(wl)


def _both(c, t, ctx, mode):
    """(logits, next) of mk_decode_step and of mk_decode_step_static for step t
    from the same cache contents, plus the static call's error record."""
    B = c.wl.run.batch
    c.reset_kv()
    c.step(t, ctx, mode)
    assert T.mk_device_error(c.q, c.ws).code == 0
    ref = (c.logits.cpu().numpy().copy(), c.nxt.cpu().numpy().copy(), c.kv_host()[0].copy())
    c.reset_kv()
    lg = torch.full_like(c.logits, float("nan"))
    nx = torch.full_like(c.nxt, -1)
    err = torch.full((8,), 0xFFFF, dtype=torch.int32, device="cuda")
    tok = torch.from_numpy(c.tokens[t].astype(np.int32)).cuda()
    cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    T.mk_decode_step_static(c.q, c.dq, c.dm.w, c.dkv.kv, tok, None, cl, B, lg, nx, err, mode)
    torch.cuda.synchronize()
    got = (lg.cpu().numpy(), nx.cpu().numpy(), c.kv_host()[0])
    return ref, got, err.cpu().numpy()


@pytest.mark.parametrize("mode", [T.MK_MEGAKERNEL, T.MK_KERNEL_PER_OP], ids=["mega", "kpo"])
def test_static_scratch_step_equals_workspace_step(mode):
    from _gpucase import log
    ncu = T.mk_get_option(T.MK_OPT_NUM_CUS)
    # first a batch of 4 over shared sub-queues, then a smaller call: batch 1, static sub-queues
    for batch, ctx0, nq in ((4, (900, 33, 500, 1023), 8), (1, (700,), ncu)):
        c = _case(batch, ctx0, nq)
        assert c.q.workspace_nbytes() <= T.MK_STATIC_SCRATCH_BYTES
        for t in range(2):
            ctx = [p + t for p in ctx0]
            ref, got, err = _both(c, t, ctx, mode)
            for a, b in zip(ref, got):
                assert np.array_equal(a, b)
            assert (err == 0).all(), err
        log(f"    static scratch, batch {batch}, mode {mode}: bit-identical to the workspace step")


def test_static_scratch_refuses_a_workspace_larger_than_the_scratch():
    """The Llama-3-8B shape at batch 16 needs about 200 MB of workspace: the call
    is refused with MK_EINVAL before anything touches the device, and a good
    call works afterwards."""
    import ctypes as C
    from tile_synchronized_decoder_amd import _lib as L
    wl = W.WORKLOADS["llama8b_b16"]
    q = T.mk_build_queue(T.make_config(wl.model), T.make_plan(wl.plan, T.MK_DECODE, 16, wl.run.ctx_max))
    assert q.workspace_nbytes() > T.MK_STATIC_SCRATCH_BYTES
    w, kv = L.mk_weights(), L.mk_kv()
    fake = C.c_void_p(0x1000)
    st = L.lib().mk_decode_step_static(q.handle, fake, C.byref(w), C.byref(kv), fake, None, fake, 16, None,
                                       None, None, T.MK_MEGAKERNEL, None)
    assert st == T.MK_EINVAL
    assert b"static scratch" in L.lib().mk_last_error()
    c = _case(1, (300,), 8)
    ref, got, err = _both(c, 0, [300], T.MK_MEGAKERNEL)
    assert all(np.array_equal(a, b) for a, b in zip(ref, got)) and (err == 0).all()
