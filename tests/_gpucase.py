"""Shared set-up of GPU parity cases: seeded inputs -> device buffers -> library
calls, and the same inputs -> float64 oracle.  Nothing here computes the decoder."""
from __future__ import annotations

import sys
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

import tile_synchronized_decoder_amd as T
from tile_synchronized_decoder_amd import device as D
import workloads as W
from oracle import numerics as N


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@dataclass
class Case:
    wl: W.Workload
    q: T.Queue
    dq: torch.Tensor
    dm: D.DeviceModel
    dkv: D.DeviceKV
    ws: torch.Tensor
    K0: np.ndarray
    V0: np.ndarray
    raw_layers: list
    raw_global: dict
    tokens: np.ndarray
    x0: Optional[np.ndarray]
    logits: Optional[torch.Tensor] = None
    nxt: Optional[torch.Tensor] = None
    model: Optional[N.Model] = None

    @property
    def m(self):
        return self.wl.model

    def oracle_model(self) -> N.Model:
        if self.model is None:
            self.model = N.prepare(self.m, self.raw_layers, self.raw_global)
        return self.model

    def reset_kv(self):
        self.dkv.k.copy_(torch.from_numpy(self.K0.view(np.int16) if self.K0.dtype == np.uint16 else self.K0))
        self.dkv.v.copy_(torch.from_numpy(self.V0.view(np.int16) if self.V0.dtype == np.uint16 else self.V0))

    def step(self, t: int, ctx: List[int], mode: int):
        """Run decode step t (teacher-forced inputs of step t) at contexts ctx."""
        m, B = self.m, self.wl.run.batch
        tok = torch.from_numpy(self.tokens[t].astype(np.int32)).cuda() if m.has_embed else None
        x0 = torch.from_numpy(self.x0[t]).cuda() if not m.has_embed else None
        cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
        T.mk_decode_step(self.q, self.dq, self.dm.w, self.dkv.kv, tok, x0, cl, B, self.ws,
                         self.logits, self.nxt, mode)
        torch.cuda.synchronize()

    def tensor(self, kind: int, layer: int, cols: int) -> np.ndarray:
        B = self.wl.run.batch
        return D.ws_view(self.ws, self.q, kind, layer, (B, cols)).cpu().numpy().astype(np.float64)

    def counters(self) -> np.ndarray:
        n = len(np.frombuffer(self.q.export(T.MK_PART_TARGETS), dtype=np.uint32))
        off = self.q.workspace_offset(T.MK_T_COUNTERS, 0)
        return self.ws[off: off + 4 * n].view(torch.int32).cpu().numpy().view(np.uint32)

    def kv_host(self):
        return D.kv_to_host(self.dkv, self.K0.dtype)


def make_case(wl: W.Workload, gain_jitter: float = 0.0, with_logits: bool = True) -> Case:
    m, r = wl.model, wl.run
    log(f"[case] {wl.name}: L={m.n_layers} H={m.hidden} V={m.vocab} B={r.batch} ctx0={r.ctx0[:4]} "
        f"ctx_max={r.ctx_max} plan={wl.plan}")
    raw_layers = W.gen.all_layer_weights(m, r.seed, gain_jitter)
    raw_global = W.gen.global_weights(m, r.seed, gain_jitter)
    K, V = W.gen.kv_cache(m, r)
    tokens = W.gen.decode_tokens(m, r)
    x0 = None if m.has_embed else W.gen.input_rows(m, r)
    q = T.mk_build_queue(T.make_config(m), T.make_plan(wl.plan, T.MK_DECODE, r.batch, r.ctx_max))
    c = Case(wl, q, D.upload_queue(q), D.upload_weights(raw_layers, raw_global), D.upload_kv(K, V),
             D.workspace(q), K, V, raw_layers, raw_global, tokens, x0)
    if m.has_lm_head and with_logits:
        c.logits = torch.zeros((r.batch, m.vocab), dtype=torch.float32, device="cuda")
        c.nxt = torch.zeros((r.batch,), dtype=torch.int32, device="cuda")
    return c
