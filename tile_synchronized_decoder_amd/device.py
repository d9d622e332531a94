"""Device memory plumbing: host arrays -> PyTorch device tensors in the layouts
include/mk.h documents (all layers of one kind stacked, [out, in] row-major;
KV cache [L][rows][n_kv][ctx_max][head_dim]).  No arithmetic happens here."""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from ._lib import mk_kv, mk_weights
from . import MK_PART_DEVICE, Queue

_MATS = ("wqkv", "wo", "wgate", "wup", "wdown")
_GAINS = ("attn_norm", "ffn_norm", "q_norm", "k_norm")


def _to_dev(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)          # bf16 bit patterns travel as int16
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


@dataclass
class DeviceModel:
    tensors: Dict[str, torch.Tensor] = field(default_factory=dict)
    w: mk_weights = field(default_factory=mk_weights)


def upload_weights(raw_layers: Sequence[Dict[str, np.ndarray]], raw_global: Dict[str, np.ndarray],
                   device="cuda") -> DeviceModel:
    dm = DeviceModel()
    for name in _MATS + _GAINS:
        if name not in raw_layers[0]:
            continue
        first = raw_layers[0][name]
        dst = torch.empty((len(raw_layers),) + first.shape,
                          dtype=torch.int16 if first.dtype == np.uint16 else torch.float32, device=device)
        for l, r in enumerate(raw_layers):
            dst[l].copy_(_to_dev(r[name], "cpu"), non_blocking=False)
        dm.tensors[name] = dst
    for name, arr in raw_global.items():
        dm.tensors[name] = _to_dev(arr, device)
    for name in _MATS + _GAINS + ("embed", "lm_head", "final_norm"):
        t = dm.tensors.get(name)
        setattr(dm.w, name, t.data_ptr() if t is not None else None)
    return dm


@dataclass
class DeviceKV:
    k: torch.Tensor
    v: torch.Tensor
    kv: mk_kv = field(default_factory=mk_kv)


def upload_kv(K: np.ndarray, V: np.ndarray, device="cuda") -> DeviceKV:
    d = DeviceKV(_to_dev(K, device), _to_dev(V, device))
    d.kv.k, d.kv.v, d.kv.rows = d.k.data_ptr(), d.v.data_ptr(), K.shape[1]
    return d


def upload_queue(q: Queue, device="cuda") -> torch.Tensor:
    """Caller-owned device copy of the queue's DEVICE image."""
    img = np.frombuffer(q.export(MK_PART_DEVICE), dtype=np.uint8)
    return torch.from_numpy(img.copy()).to(device)


def workspace(q: Queue, device="cuda") -> torch.Tensor:
    return torch.zeros(q.workspace_nbytes(), dtype=torch.uint8, device=device)


def ws_view(ws: torch.Tensor, q: Queue, tensor: int, layer: int, shape) -> torch.Tensor:
    """fp32 view of one workspace tensor (device)."""
    off = q.workspace_offset(tensor, layer)
    n = int(np.prod(shape))
    return ws[off: off + 4 * n].view(torch.float32).view(*shape)


def kv_to_host(d: DeviceKV, dtype) -> tuple:
    k = d.k.cpu().numpy()
    v = d.v.cpu().numpy()
    if dtype == np.uint16:
        return k.view(np.uint16), v.view(np.uint16)
    return k, v
