"""Tile-synchronized decoder megakernel for MI355X: thin Python binding of libmk.so.

The names match the C ABI (include/mk.h).  These wrappers only marshal
arguments: device memory and streams come from PyTorch (tensors' data
pointers, the current stream), all computation runs in the library's HIP
kernels, and a missing library raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Dict, Optional

from . import _lib as _L
from ._lib import (MK_OK, MK_EINVAL, MK_ENOMEM, MK_ELAUNCH, MK_EDEVICE, MK_ENOTSUP,
                   MK_BF16, MK_DECODE, MK_F32, MK_KERNEL_PER_OP, MK_KERNEL_PER_OP_GRAPH, MK_MEGAKERNEL, MK_MULTI_STREAM, MK_PREFILL,
                   MK_PART_DEVICE, MK_PART_INSTR, MK_PART_META, MK_PART_TARGETS, MK_PART_WAITS, MK_STATIC_SCRATCH_BYTES,
                   MK_T_ACT, MK_T_ATT, MK_T_COUNTERS, MK_T_ERROR, MK_T_HEADS, MK_T_HRES,
                   MK_T_OPART, MK_T_QKV, MK_T_X, MK_OPT_NUM_CUS, MK_OPT_SPIN_LIMIT, MK_OPT_TRACE_BUFFER,
                   MK_OPT_TRACE_BYTES, MK_OPT_GEMV_PIPE, MK_OPT_DELAY_SEED, MK_OPT_STREAMS,
                   MK_OPT_MEGAKERNELS, MK_OPT_PREFILL_LO,
                   MK_OPT_WORKERS_PER_CU, MkError, mk_config, mk_dev_error, mk_kv, mk_plan,
                   mk_weights)

PART_NAMES = {"meta": MK_PART_META, "instr": MK_PART_INSTR, "waits": MK_PART_WAITS,
              "targets": MK_PART_TARGETS}


def make_config(model) -> mk_config:
    """mk_config from any object with the ModelConfig attribute names."""
    return mk_config(model.n_layers, model.hidden, model.n_q_heads, model.n_kv_heads,
                     model.head_dim, model.ffn, model.vocab, int(model.qk_norm),
                     int(model.has_embed), int(model.has_lm_head),
                     MK_BF16 if model.dtype == "bf16" else MK_F32, model.rms_eps, model.rope_theta)


def make_plan(plan, mode: int, rows: int, ctx_max: int) -> mk_plan:
    return mk_plan(mode, rows, ctx_max, plan.tq, plan.to, plan.tf, plan.td, plan.kb, plan.bm,
                   plan.bn, plan.n_queues, getattr(plan, "fuse_combine", 0), getattr(plan, "loop", 0),
                   getattr(plan, "attn_pop", 0))


class Queue:
    """Owns a host mk_queue handle."""

    def __init__(self, handle: int, cfg: mk_config, plan: mk_plan):
        self.handle = C.c_void_p(handle)
        self.cfg, self.plan = cfg, plan

    def nbytes(self, part: int) -> int:
        return _L.lib().mk_queue_nbytes(self.handle, part)

    def export(self, part: int) -> bytes:
        n = self.nbytes(part)
        buf = (C.c_uint8 * max(n, 1))()
        _L.check(_L.lib().mk_queue_export(self.handle, part, buf, n), "mk_queue_export")
        return bytes(buf[:n])

    def parts(self) -> Dict[str, bytes]:
        return {name: self.export(p) for name, p in PART_NAMES.items()}

    def workspace_nbytes(self) -> int:
        n = C.c_size_t()
        _L.check(_L.lib().mk_workspace_nbytes(self.handle, C.byref(n)), "mk_workspace_nbytes")
        return n.value

    def workspace_offset(self, tensor: int, layer: int = 0) -> int:
        n = C.c_size_t()
        _L.check(_L.lib().mk_workspace_offset(self.handle, tensor, layer, C.byref(n)),
                 "mk_workspace_offset")
        return n.value

    def close(self) -> None:
        if self.handle:
            _L.lib().mk_queue_free(self.handle)
            self.handle = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:       # noqa: BLE001 -- interpreter shutdown
            pass


def mk_build_queue(cfg: mk_config, plan: mk_plan) -> Queue:
    h = C.c_void_p()
    _L.check(_L.lib().mk_build_queue(C.byref(cfg), C.byref(plan), C.byref(h)), "mk_build_queue")
    return Queue(h.value, cfg, plan)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def mk_decode_step(q: Queue, d_queue, w: mk_weights, kv: mk_kv, tokens, x0, ctx_lens, batch: int,
                   workspace, logits, next_tokens, exec_mode: int = MK_MEGAKERNEL, stream=None) -> None:
    _L.check(_L.lib().mk_decode_step(q.handle, _ptr(d_queue), C.byref(w), C.byref(kv), _ptr(tokens),
                                     _ptr(x0), _ptr(ctx_lens), batch, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _ptr(logits),
                                     _ptr(next_tokens), exec_mode, _stream(stream)), "mk_decode_step")


def mk_decode_step_static(q: Queue, d_queue, w: mk_weights, kv: mk_kv, tokens, x0, ctx_lens, batch: int,
                          logits, next_tokens, error=None, exec_mode: int = MK_MEGAKERNEL, stream=None) -> None:
    """mk_decode_step on the library's static device scratch (no workspace)."""
    _L.check(_L.lib().mk_decode_step_static(q.handle, _ptr(d_queue), C.byref(w), C.byref(kv), _ptr(tokens),
                                            _ptr(x0), _ptr(ctx_lens), batch, _ptr(logits), _ptr(next_tokens),
                                            _ptr(error), exec_mode, _stream(stream)), "mk_decode_step_static")


def mk_decode_loop(q: Queue, d_queue, w: mk_weights, kv: mk_kv, tokens, ctx_lens, batch: int, steps: int,
                   feedback: int, workspace, logits, next_tokens, stream=None) -> None:
    """`steps` decode steps of a loop queue in one launch (see include/mk.h)."""
    _L.check(_L.lib().mk_decode_loop(q.handle, _ptr(d_queue), C.byref(w), C.byref(kv), _ptr(tokens),
                                     _ptr(ctx_lens), batch, steps, feedback, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _ptr(logits),
                                     _ptr(next_tokens), _stream(stream)), "mk_decode_loop")


def mk_lm_head(q: Queue, w: mk_weights, workspace, logits, next_tokens, stream=None) -> None:
    _L.check(_L.lib().mk_lm_head(q.handle, C.byref(w), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _ptr(logits),
                                 _ptr(next_tokens), _stream(stream)), "mk_lm_head")


def mk_prefill(q: Queue, d_queue, w: mk_weights, kv: mk_kv, tokens, seq_len: int, kv_row: int,
               workspace, logits_last, next_tokens, exec_mode: int = MK_MEGAKERNEL, stream=None) -> None:
    _L.check(_L.lib().mk_prefill(q.handle, _ptr(d_queue), C.byref(w), C.byref(kv), _ptr(tokens),
                                 seq_len, kv_row, _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _ptr(logits_last),
                                 _ptr(next_tokens), exec_mode, _stream(stream)), "mk_prefill")


def mk_device_error(q: Queue, workspace, stream=None) -> mk_dev_error:
    """Synchronises the stream; returns the device error record (code 0 = none)."""
    e = mk_dev_error()
    st = _L.lib().mk_device_error(q.handle, _ptr(workspace), C.byref(e), _stream(stream))
    if st not in (_L.MK_OK, _L.MK_EDEVICE):
        _L.check(st, "mk_device_error")
    return e


def mk_set_option(key: int, value: int) -> None:
    _L.check(_L.lib().mk_set_option(key, value), "mk_set_option")


def mk_get_option(key: int) -> int:
    return int(_L.lib().mk_get_option(key))


def library_path() -> str:
    return _L.LIB_PATH
