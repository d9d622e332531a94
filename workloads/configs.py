"""Workload definitions: model shapes, run shapes and default tile plans.

These are plain parameter tables.  They hold none of the decoder's arithmetic:
the CPU oracle and the GPU library both receive the same values from here.

The five workloads follow the decoder shapes the megakernel pages evaluate on
(dense Llama-3 and Qwen3 models, MegaOps abstract; Llama-1B in the "One
Megakernel is Not Enough" abstract), at random initialisation:

* ``layer256_f32``       one Llama-style layer, fp32, hidden 256, GQA 4/2, FFN 688
* ``llama1b_b1``         Llama-3-1B-shaped, bf16, batch 1, 128 steps from a 1024-token cache
* ``llama8b_b{1,4,16}``  Llama-3-8B-shaped, bf16, context 4096
* ``qwen8b_prefill``     Qwen3-8B-shaped with per-head QK RMSNorm, 2048-token prefill then 64 steps
* ``llama1b_stream_b32`` Llama-3-1B-shaped, batch 32, per-sequence contexts U{256..8192}, 256 steps
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional, Tuple

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int            # 0 when the model has neither embedding nor LM head
    rms_eps: float
    rope_theta: float
    qk_norm: bool = False
    dtype: str = BF16     # storage type of matrices and of the KV cache
    has_embed: bool = True
    has_lm_head: bool = True

    @property
    def group(self) -> int:          # query heads per KV head
        return self.n_q_heads // self.n_kv_heads

    @property
    def qkv_cols(self) -> int:       # rows of the stacked [q | k | v] projection
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def attn_cols(self) -> int:
        return self.n_q_heads * self.head_dim


@dataclass(frozen=True)
class Plan:
    """Tile parameters of the instruction queue (explicit inputs, never inferred).

    tq/to/tf/td: output-column tile widths of the QKV, O-projection, gate/up and
    down GEMVs.  kb: keys per attention split.  bm/bn: prefill GEMM tile.
    n_queues: number of sub-queues the workers pop from (instruction i belongs to
    sub-queue i mod n_queues).
    fuse_combine: decode only; 1 drops the split-combine instructions: each
    O-projection tile waits on the attention splits' partials and merges them
    itself while staging its inputs (one barrier hand-off fewer per layer).
    2 drops them too: the split that completes a (row, KV head) merges its
    partials into the attention output and signals the partial tile once more
    (target NS + 1), and the O-projection tiles wait on those tiles.
    prefill_queues: sub-queues of the prefill queue (0: n_queues).  Prefill
    instructions are long, so shared sub-queues (workers pop dynamically) cost
    little and balance the causal attention tiles' unequal lengths.
    loop: decode only; 1 builds a queue for persistent multi-step decode: each
    step ends with LM-head tiles (64 vocabulary rows each) and one argmax per
    row, and the next step's embedding tiles wait on the previous step's argmax.
    attn_pop: decode only, single-step queues; 1 hands a layer's attention
    splits out at run time in the megakernel (workers take them from a
    per-layer counter), so that ragged contexts load the workers evenly.
    """
    tq: int = 16
    to: int = 16
    tf: int = 16
    td: int = 16
    kb: int = 256
    bm: int = 128
    bn: int = 128
    n_queues: int = 1
    fuse_combine: int = 0
    prefill_queues: int = 0
    loop: int = 0
    attn_pop: int = 0

    def for_prefill(self) -> "Plan":
        """The plan of the prefill queue (its own sub-queue count)."""
        return dataclasses.replace(self, n_queues=self.prefill_queues or self.n_queues, loop=0)


@dataclass(frozen=True)
class RunConfig:
    batch: int                       # B (decode rows)
    ctx0: Tuple[int, ...]            # cached positions per sequence before step 0
    steps: int                       # teacher-forced decode steps
    ctx_max: int                     # allocated cache positions per sequence
    seed: int
    prefill_len: int = 0             # tokens prefilled before decoding (cache empty before)
    init_cache: bool = True          # random N(0,1) cache entries below ctx0


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelConfig
    run: RunConfig
    plan: Plan = field(default_factory=Plan)
    describe: str = ""


LLAMA_LAYER_F32 = ModelConfig(
    name="llama-layer-h256-f32", n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2,
    head_dim=64, ffn=688, vocab=0, rms_eps=1e-5, rope_theta=1e4, dtype=F32,
    has_embed=False, has_lm_head=False)

LLAMA_1B = ModelConfig(
    name="llama3-1b-shaped", n_layers=16, hidden=2048, n_q_heads=32, n_kv_heads=8,
    head_dim=64, ffn=8192, vocab=128256, rms_eps=1e-5, rope_theta=5e5)

LLAMA_8B = ModelConfig(
    name="llama3-8b-shaped", n_layers=32, hidden=4096, n_q_heads=32, n_kv_heads=8,
    head_dim=128, ffn=14336, vocab=128256, rms_eps=1e-5, rope_theta=5e5)

QWEN_8B = ModelConfig(
    name="qwen3-8b-shaped", n_layers=36, hidden=4096, n_q_heads=32, n_kv_heads=8,
    head_dim=128, ffn=12288, vocab=151936, rms_eps=1e-6, rope_theta=1e6, qk_norm=True)


# Plans of the benchmark workloads: one sub-queue per worker of an MI355X (256
# compute units) and tile widths that give each GEMV op about 256 tiles.  At
# batch 1 the last-arriving split merges the attention partials (fuse_combine
# 2: one stage and barrier hop fewer per layer, 1% faster); with more rows
# there are rows x KV heads merges per layer, which then land on the workers
# whose splits end last, and separate combine tiles spread over all workers
# are faster (5-19% at batch 4 to 32).  With several rows the split size
# is chosen so that rows x KV heads x splits about fills the 256 workers once
# (8B at context 4224: 576 keys at batch 4, 2112 at batch 16): per-split work
# (waiting, staging q, merging lane groups, writing partials) then repeats
# fewer times per row; at batch 1 the 256-key splits keep their 1-round
# balance with merges in the last split.  At batch 32 with ragged contexts
# (256..8192 keys) the splits are handed out at run time and sized at 6144
# keys: most (row, KV head) pairs are one split, so each row's attention pays
# its fixed work and merge once; measured over 64 steps, 3.73 ms per step
# against 3.89 (3072-key splits) and 4.07 (2048), the per-op kernels 3.78,
# 3.79 and 3.84 on the same queues.
PLAN_8B = Plan(tq=24, to=16, tf=56, td=16, n_queues=256)
PLAN_8B_B1 = dataclasses.replace(PLAN_8B, fuse_combine=2)
PLAN_8B_B4 = dataclasses.replace(PLAN_8B, kb=576)
PLAN_8B_B16 = dataclasses.replace(PLAN_8B, kb=2112)


def _stream_ctx0(seed: int, batch: int, lo: int, hi: int) -> Tuple[int, ...]:
    # per-sequence starting contexts, uniform integers in [lo, hi], seeded
    import numpy as np
    ss = np.random.SeedSequence(seed, spawn_key=(7, 0, 0))
    g = np.random.Generator(np.random.PCG64(ss))
    return tuple(int(v) for v in g.integers(lo, hi + 1, size=batch))


WORKLOADS = {
    "layer256_f32": Workload(
        "layer256_f32", LLAMA_LAYER_F32,
        RunConfig(batch=1, ctx0=(128,), steps=1, ctx_max=129, seed=1),
        Plan(tq=16, to=16, tf=32, td=16, kb=32),
        "single fp32 Llama-style layer, hidden 256, GQA 4/2, FFN 688, one step at position 128"),
    "llama1b_b1": Workload(
        "llama1b_b1", LLAMA_1B,
        RunConfig(batch=1, ctx0=(1024,), steps=128, ctx_max=1152, seed=2),
        Plan(tf=32, td=8, n_queues=256, fuse_combine=2),
        "Llama-3-1B-shaped bf16, batch 1, 128 decode steps from a 1024-token cache"),
    "llama8b_b1": Workload(
        "llama8b_b1", LLAMA_8B,
        RunConfig(batch=1, ctx0=(4096,), steps=128, ctx_max=4224, seed=3), PLAN_8B_B1,
        "Llama-3-8B-shaped bf16, batch 1, context 4096"),
    "llama8b_b4": Workload(
        "llama8b_b4", LLAMA_8B,
        RunConfig(batch=4, ctx0=(4096,) * 4, steps=128, ctx_max=4224, seed=3), PLAN_8B_B4,
        "Llama-3-8B-shaped bf16, batch 4, context 4096"),
    "llama8b_b16": Workload(
        "llama8b_b16", LLAMA_8B,
        RunConfig(batch=16, ctx0=(4096,) * 16, steps=128, ctx_max=4224, seed=3), PLAN_8B_B16,
        "Llama-3-8B-shaped bf16, batch 16, context 4096"),
    "qwen8b_prefill": Workload(
        "qwen8b_prefill", QWEN_8B,
        RunConfig(batch=1, ctx0=(2048,), steps=64, ctx_max=2112, seed=4, prefill_len=2048,
                  init_cache=False), Plan(tq=24, to=16, tf=48, td=16, n_queues=256, prefill_queues=8,
                                          fuse_combine=2),
        "Qwen3-8B-shaped bf16 with QK-norm: prefill of 2048 tokens, then 64 decode steps"),
    "llama1b_stream_b32": Workload(
        "llama1b_stream_b32", LLAMA_1B,
        RunConfig(batch=32, ctx0=_stream_ctx0(5, 32, 256, 8192), steps=256, ctx_max=8448, seed=5),
        Plan(tf=32, td=8, kb=6144, n_queues=256, attn_pop=1),
        "Llama-3-1B-shaped bf16 streaming decode, batch 32, contexts U{256..8192}, 256 steps"),
}


def shrink(w: Workload, *, n_layers: Optional[int] = None, vocab: Optional[int] = None,
           batch: Optional[int] = None, ctx0: Optional[Tuple[int, ...]] = None,
           ctx_max: Optional[int] = None, steps: Optional[int] = None,
           name: Optional[str] = None) -> Workload:
    """A copy of ``w`` with fewer layers / smaller vocab / other run shape, for
    tests that must stay within seconds on the CPU."""
    m = w.model
    if n_layers is not None or vocab is not None:
        m = dataclasses.replace(m, n_layers=n_layers if n_layers is not None else m.n_layers,
                                vocab=vocab if vocab is not None else m.vocab)
    r = w.run
    kw = {}
    if batch is not None:
        kw["batch"] = batch
    if ctx0 is not None:
        kw["ctx0"] = tuple(ctx0)
    if ctx_max is not None:
        kw["ctx_max"] = ctx_max
    if steps is not None:
        kw["steps"] = steps
    if kw:
        r = dataclasses.replace(r, **kw)
    return Workload(name or w.name, m, r, w.plan, w.describe)
