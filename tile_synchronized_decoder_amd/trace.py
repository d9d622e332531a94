"""Megakernel trace: per-instruction timestamps -> per-op statistics and a
Chrome trace (chrome://tracing / Perfetto) with one track per workgroup.

Usage with the binding:
    buf = torch.zeros(8 * n_instr, dtype=torch.int64, device="cuda")
    mk_set_option(MK_OPT_TRACE_BYTES, buf.numel() * 8)
    mk_set_option(MK_OPT_TRACE_BUFFER, buf.data_ptr())
    ... one mk_decode_step ...
    mk_set_option(MK_OPT_TRACE_BUFFER, 0)
    records = parse(buf.cpu().numpy(), instr_bytes)
"""
from __future__ import annotations

import json
from typing import Dict, List

import numpy as np

OP_NAMES = {1: "EMBED", 2: "QKV", 3: "ATTN", 4: "COMBINE", 5: "OPROJ", 6: "GATEUP", 7: "DOWN",
            8: "P_EMBED", 9: "P_QKV", 10: "P_ATTN", 11: "P_OPROJ", 12: "P_GATEUP", 13: "P_DOWN"}
TICK_US = 0.01          # the device wall clock runs at 100 MHz
WORDS = 8               # u64 per instruction record


def parse(trace: np.ndarray, instr_bytes: bytes) -> np.ndarray:
    """Structured records: idx, op, layer, workgroup, xcd, start, ready, phase_a, phase_b,
    end (microseconds from the first pop).  Instructions without a wait list have
    ready = start; a phase an op does not mark is NaN."""
    t = np.asarray(trace, dtype=np.uint64).reshape(-1, WORDS)
    rec = np.frombuffer(instr_bytes, dtype=np.dtype([("op", "<u2"), ("layer", "<u2"), ("f", "<u4", (7,))]))
    n = len(rec)
    t = t[:n]
    start = t[:, 1].astype(np.int64)
    t0 = start[start > 0].min()
    ready = np.where(t[:, 2] > 0, t[:, 2].astype(np.int64), start)
    out = np.zeros(n, dtype=[("idx", "i4"), ("op", "i4"), ("layer", "i4"), ("wg", "i4"), ("xcd", "i4"),
                             ("start", "f8"), ("ready", "f8"), ("phase_a", "f8"), ("phase_b", "f8"),
                             ("end", "f8")])
    out["idx"] = np.arange(n)
    out["op"] = rec["op"]
    out["layer"] = rec["layer"]
    out["wg"] = (t[:, 0] >> np.uint64(32)).astype(np.int64)
    out["xcd"] = (t[:, 0] & np.uint64(0xF)).astype(np.int64)
    out["start"] = (start - t0) * TICK_US
    out["ready"] = (ready - t0) * TICK_US
    for name, col in (("phase_a", 3), ("phase_b", 4)):
        v = t[:, col].astype(np.int64)
        out[name] = np.where(v > 0, (v - t0) * TICK_US, np.nan)
    out["end"] = (t[:, 5].astype(np.int64) - t0) * TICK_US
    return out


def op_stats(r: np.ndarray) -> Dict[str, Dict[str, float]]:
    """Mean times per opcode, in microseconds: wait (pop -> waits ended), run (waits
    ended -> end), and the run split into stage (-> phase A), loop (A -> B) and
    tail (B -> end) where the op marks its phases."""
    stats = {}
    for op in np.unique(r["op"]):
        m = r[r["op"] == op]
        st = {"count": int(len(m)), "wait_us": float(np.mean(m["ready"] - m["start"])),
              "run_us": float(np.mean(m["end"] - m["ready"]))}
        a, b = m["phase_a"], m["phase_b"]
        if np.isfinite(a).any():
            st["stage_us"] = float(np.nanmean(a - m["ready"]))
        if np.isfinite(b).any():
            st["loop_us"] = float(np.nanmean(b - np.where(np.isfinite(a), a, m["ready"])))
            st["tail_us"] = float(np.nanmean(m["end"] - b))
        st["first_start_us"] = float(m["start"].min())
        st["last_end_us"] = float(m["end"].max())
        stats[OP_NAMES.get(int(op), str(op))] = st
    return stats


def layer_spans(r: np.ndarray) -> List[Dict[str, float]]:
    """Per layer and op: when its first instruction started and its last one ended."""
    out = []
    for l in np.unique(r["layer"]):
        for op in np.unique(r["op"]):
            m = r[(r["layer"] == l) & (r["op"] == op)]
            if len(m):
                out.append({"layer": int(l), "op": OP_NAMES.get(int(op), str(op)),
                            "start": float(m["start"].min()), "ready_last": float(m["ready"].max()),
                            "end": float(m["end"].max())})
    return out


def chrome_trace(r: np.ndarray) -> str:
    ev = []
    for x in r:
        name = f"{OP_NAMES.get(int(x['op']), x['op'])} L{x['layer']} #{x['idx']}"
        ev.append({"name": "wait", "ph": "X", "pid": int(x["xcd"]), "tid": int(x["wg"]),
                   "ts": float(x["start"]), "dur": float(x["ready"] - x["start"])})
        ev.append({"name": name, "ph": "X", "pid": int(x["xcd"]), "tid": int(x["wg"]),
                   "ts": float(x["ready"]), "dur": float(x["end"] - x["ready"])})
    return json.dumps({"traceEvents": ev})
