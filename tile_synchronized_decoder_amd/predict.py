"""Step-time predictor for a megakernel queue: one event pass over its tile graph.

The "One Megakernel is Not Enough" abstract (arXiv 2610.35336) chooses where to
cut a model into megakernels from conventional-graph profiles and standalone
kernel timings, by simulating each candidate's tile and event graphs instead of
running it.  This module does that for the two designs this library runs: the
whole decode step as one megakernel, or one kernel per operator.

What the queue fixes (the layout of mk_build_queue's parts):
  * instruction i runs on worker i mod n_queues (one worker per sub-queue when
    the queue has as many sub-queues as the grid has workgroups), in queue order;
  * it waits on ranges of tile barriers and signals one barrier; a barrier is
    complete once all instructions that signal it (its target) have ended.

Every barrier an instruction waits on is signalled only by earlier instructions
(queue order is topological; the CPU checker verifies it), and a worker's
previous instruction is earlier as well, so start and end times follow in a
single pass in queue order.  Per instruction i on worker w:

    free  = end of w's previous instruction (0 for its first)
    ready = max over waited barriers b of done[b] + hop     (free if it waits on none)
    lead  = min(prefetch[op], max(0, ready - free), dur[op])   (streamed while waiting)
    end   = max(free, ready) + dur[op] - lead
    done[signal] = max(done[signal], end)

dur[op] is one instruction's run time, hop the time from a producer's signal to
a consumer seeing it and holding its inputs, prefetch[op] how much of an
instruction's streaming fits the shared-memory ring it fills before it waits.
The predicted step is the last end.  With kernel-per-op the same instructions
run op by op, each op one launch whose time is a measured kernel time.

Host only; no device code.  Inputs are the queue's exported parts and timings
in microseconds.
"""
from __future__ import annotations

import re
import struct
from dataclasses import dataclass
from typing import Dict, List, Mapping, Optional, Sequence, Tuple

import numpy as np

OP_NAMES = {1: "EMBED", 2: "QKV", 3: "ATTN", 4: "COMBINE", 5: "OPROJ", 6: "GATEUP", 7: "DOWN"}


@dataclass
class Graph:
    """The tile graph of a queue: per instruction op, layer, wait ranges and signal."""
    op: np.ndarray            # [n] int
    layer: np.ndarray         # [n] int
    wait_off: np.ndarray      # [n] first wait range
    wait_cnt: np.ndarray      # [n] number of wait ranges
    signal: np.ndarray        # [n] barrier signalled
    ranges: np.ndarray        # [n_ranges, 2] (first barrier, count)
    targets: np.ndarray       # [n_barriers]
    n_queues: int


def graph_from_parts(parts: Mapping[str, bytes]) -> Graph:
    """Decode the META, INSTR, WAITS and TARGETS parts of an exported queue."""
    meta = parts["meta"]
    if meta[:4] != b"TMK1":
        raise ValueError("not a queue META part")
    n_queues = struct.unpack_from("<I", meta, 4 * 7)[0]
    rec = np.frombuffer(parts["instr"], dtype="<u4").reshape(-1, 8)
    return Graph(op=(rec[:, 0] & 0xFFFF).astype(np.int64), layer=(rec[:, 0] >> 16).astype(np.int64),
                 wait_off=rec[:, 4].astype(np.int64), wait_cnt=rec[:, 5].astype(np.int64),
                 signal=rec[:, 6].astype(np.int64),
                 ranges=np.frombuffer(parts["waits"], dtype="<u4").reshape(-1, 2).astype(np.int64),
                 targets=np.frombuffer(parts["targets"], dtype="<u4").astype(np.int64),
                 n_queues=int(n_queues))


def simulate(g: Graph, dur: Mapping[int, float], hop: float = 0.0,
             prefetch: Optional[Mapping[int, float]] = None,
             n_workers: Optional[int] = None) -> Tuple[float, np.ndarray, np.ndarray]:
    """Event pass over the schedule.  Returns (step, start, end) in the units of
    `dur`.  With as many workers as sub-queues (the default) instruction i runs
    on worker i mod n_queues.  With more workers than sub-queues, the workers
    w, w + n_queues, ... share sub-queue w mod n_queues and pop from it in
    order: each instruction goes to the one of them that is free first."""
    nq = g.n_queues
    nw = n_workers or nq
    prefetch = prefetch or {}
    n = len(g.op)
    start = np.zeros(n)
    end = np.zeros(n)
    done = np.zeros(len(g.targets))
    free = np.zeros(nw)
    # the workers of each sub-queue (a worker beyond the queue count shares one)
    members = [np.arange(q, nw, nq) for q in range(min(nq, nw))] if nw > nq else None
    rng = g.ranges
    for i in range(n):
        if members is None:
            w = i % nw
        else:
            mq = members[i % nq]
            w = int(mq[np.argmin(free[mq])])
        f = free[w]
        ready = f
        o, c = g.wait_off[i], g.wait_cnt[i]
        if c:
            t = max(done[rng[k, 0]:rng[k, 0] + rng[k, 1]].max() for k in range(o, o + c)) + hop
            ready = max(ready, t)
        op = int(g.op[i])
        d = dur[op]
        lead = min(prefetch.get(op, 0.0), max(0.0, ready - f), d)
        s = max(f, ready)
        e = s + d - lead
        start[i], end[i] = s, e
        free[w] = e
        sg = g.signal[i]
        if e > done[sg]:
            done[sg] = e
    return (float(end.max()) if n else 0.0), start, end


def op_counts(g: Graph) -> Dict[int, int]:
    """Instructions per op per layer (the op's per-op launch size)."""
    out: Dict[int, int] = {}
    nl = int(g.layer.max()) + 1 if len(g.layer) else 1
    for op in np.unique(g.op):
        out[int(op)] = int((g.op == op).sum()) // (nl if op != 1 else 1)
    return out


def per_instruction_us(kernel_us: Mapping[int, float], counts: Mapping[int, int], n_cus: int) -> Dict[int, float]:
    """One instruction's run time from a per-op kernel's time: a launch of n
    instructions runs ceil(n / n_cus) rounds of concurrent workgroups."""
    return {op: kernel_us[op] / max(1, -(-counts[op] // n_cus)) for op in kernel_us}


def kpo_step(g: Graph, kernel_us: Mapping[int, float], gap_us: float) -> float:
    """Kernel-per-op step: every (layer, op) launch in turn, plus a launch gap each."""
    n_launch = 0
    total = 0.0
    seen = set()
    for op, layer in zip(g.op.tolist(), g.layer.tolist()):
        if (op, layer) in seen:
            continue
        seen.add((op, layer))
        total += kernel_us[op]
        n_launch += 1
    return total + n_launch * gap_us


_KPO_NAME = re.compile(r"kpo_kernel<[^,]+,\s*\d+,\s*(\d+)>")


def kpo_kernel_us(stats_rows: Sequence[Tuple[str, float]]) -> Dict[int, float]:
    """Average per-op kernel times (µs) from (kernel name, average ns) rows of a
    rocprofv3 kernel-stats table; the fused O-projection variant counts as OPROJ."""
    out: Dict[int, float] = {}
    for name, avg_ns in stats_rows:
        m = _KPO_NAME.search(name)
        if m:
            op = int(m.group(1))
            out[5 if op == 100 else op] = avg_ns / 1000.0
    return out


def read_kernel_stats_csv(path: str) -> List[Tuple[str, float]]:
    """(name, average ns) rows of a rocprofv3 --stats kernel_stats.csv file."""
    import csv
    with open(path) as f:
        return [(r["Name"], float(r["AverageNs"])) for r in csv.DictReader(f)]


def read_kernel_stats_md(path: str) -> List[Tuple[str, float]]:
    """(name, average ns) rows of a kernel-time summary table (kernel, calls,
    avg (us), ...) as the profiling module writes it."""
    out = []
    with open(path) as f:
        for line in f:
            if line.startswith("| `"):
                cells = [c.strip() for c in line.strip().strip("|").split("|")]
                out.append((cells[0].strip("`"), float(cells[2]) * 1000.0))
    return out


def gemv_prefetch_us(dur: Mapping[int, float], weight_bytes: Mapping[int, int], ring_bytes: int) -> Dict[int, float]:
    """Time's worth of a GEMV instruction's weights that its ring holds before it
    waits: the ring's share of the instruction's weight bytes, times its run time."""
    return {op: min(1.0, ring_bytes / b) * dur[op] for op, b in weight_bytes.items() if op in dur}


def main():
    import argparse
    import tile_synchronized_decoder_amd as T
    import workloads as W
    ap = argparse.ArgumentParser(description="predict the megakernel decode step from per-op kernel times")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--stats", required=True, help="kernel-time summary (.md) or rocprofv3 kernel_stats.csv "
                                                   "holding the per-op kernels of that workload")
    ap.add_argument("--hop", type=float, default=1.0, help="barrier hand-off, µs")
    ap.add_argument("--cus", type=int, default=256)
    a = ap.parse_args()
    wl = W.WORKLOADS[a.workload]
    m, r, p = wl.model, wl.run, wl.plan
    q = T.mk_build_queue(T.make_config(m), T.make_plan(p, T.MK_DECODE, r.batch, r.ctx_max))
    g = graph_from_parts(q.parts())
    rows = read_kernel_stats_md(a.stats) if a.stats.endswith(".md") else read_kernel_stats_csv(a.stats)
    kern = kpo_kernel_us(rows)
    dur = per_instruction_us(kern, op_counts(g), a.cus)
    es = 2 if m.dtype == "bf16" else 4
    na = m.n_q_heads * m.head_dim
    wbytes = {2: p.tq * m.hidden * es, 5: p.to * na * es, 6: 2 * p.tf * m.hidden * es, 7: p.td * m.ffn * es}
    ring = 4 * (20 if r.batch <= 2 else 16) * 1024          # four waves' weight rings (1 KB lines)
    nw = a.cus if g.n_queues < a.cus else None
    step, _, _ = simulate(g, dur, a.hop, gemv_prefetch_us(dur, wbytes, ring), n_workers=nw)
    kpo = kpo_step(g, kern, 0.0)
    mega = [avg / 1000.0 for name, avg in rows if "mk_interp<" in name]
    line = {"workload": a.workload, "predicted_megakernel_us": round(step, 1), "kernel_per_op_sum_us": round(kpo, 1),
            "pick": "megakernel" if step < kpo else "kernel-per-op"}
    if mega:
        line["measured_megakernel_us"] = round(mega[0], 1)
        line["error_pct"] = round(100 * (step / mega[0] - 1), 1)
        line["measured_pick"] = "megakernel" if mega[0] < kpo else "kernel-per-op"
    import json
    print(json.dumps(line))


if __name__ == "__main__":
    main()
