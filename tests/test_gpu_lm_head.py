"""The separate LM-head kernels on the GPU against the float64 oracle.

mk_lm_head normalises the workspace's last hidden rows and multiplies them by
the LM-head matrix.  Up to 4 rows stream the weights through registers where
the normalised rows fit in 64 KB of shared memory; otherwise up to 32 rows of
bf16 weights run on the matrix cores with the normalised rows split into bf16
hi and lo parts (5 to 32 rows of the 1B shape, 4 rows of the 8B one; its 2
rows still take the register kernel).  Both must match the oracle's fp64 logits to fp32
accuracy (2e-5 per row here, against the model-level 2e-2), with a vocabulary
that ends inside a 64-row block and inside a 512-row workgroup, and the argmax
must be the lowest index of the largest logit.
"""
import numpy as np
import pytest
import torch

import tile_synchronized_decoder_amd as T
from tile_synchronized_decoder_amd import device as D
import workloads as W
from oracle import numerics as N

pytestmark = pytest.mark.gpu

TOL = 2e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("base,rows", [("llama1b_b1", 1), ("llama1b_b1", 4), ("llama1b_b1", 5), ("llama1b_b1", 8),
                                       ("llama1b_b1", 17), ("llama1b_b1", 32), ("llama8b_b1", 2),
                                       ("llama8b_b1", 4)])
def test_lm_head_matches_oracle(base, rows):
    from _gpucase import make_case, log
    wl = W.shrink(W.WORKLOADS[base], n_layers=1, vocab=4136, batch=rows, ctx0=(100,) * rows, steps=1,
                  name=f"{base}_L1_V4136_B{rows}")
    c = make_case(wl, gain_jitter=0.1)
    m = c.m
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(77, spawn_key=(rows,))))
    x = g.standard_normal((rows, m.hidden)).astype(np.float32)
    x[0] *= 3.0                                               # rows of different scales
    D.ws_view(c.ws, c.q, T.MK_T_X, m.n_layers, (rows, m.hidden)).copy_(torch.from_numpy(x))
    lg = torch.full((rows, m.vocab), float("nan"), dtype=torch.float32, device="cuda")
    nx = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    T.mk_lm_head(c.q, c.dm.w, c.ws, lg, nx)
    torch.cuda.synchronize()
    got = lg.cpu().numpy()
    model = c.oracle_model()
    ref = N.lm_head(m, x.astype(np.float64), model.final_norm, model.lm_head)
    e = N.max_rel_err_rows(got.astype(np.float64), ref)
    log(f"    LM head, {rows} rows, vocab {m.vocab}: max row error {e:.2e}")
    assert np.isfinite(got).all()
    assert e <= TOL, e
    assert np.array_equal(nx.cpu().numpy(), N.argmax_lowest(got))
