"""Step-time predictor: one event pass over a queue's tile graph per design.

The "One Megakernel is Not Enough" abstract chooses how to cut a model into
kernels from standalone kernel timings, by simulating each candidate's tile
and event graphs instead of running it, and checks the picks against
measurement.  This module does that for the designs this library runs:

* ``mega``       the decode step as one persistent megakernel, then the LM
                 head and argmax as separate kernels;
* ``loop``       the LM head and argmax inside the megakernel (a loop queue,
                 several steps per launch): the LM-head placement question;
* ``kpo``        one kernel per (layer, op) segment in stream order, eager;
* ``kpo_graph``  the same launches replayed from a HIP graph;
* ``msS``        one kernel per segment on S streams, synchronised on tiles;
* ``megaK``      a composition of K megakernels per step, cut at layer
                 boundaries (launch k runs layers [k L / K, (k + 1) L / K)).

Inputs, all measured on their own: the per-op kernels of the kernel-per-op
mode (one launch per op: rocprofv3 kernel statistics), the separate LM-head,
argmax and counter-reset kernels, and the host's time to enqueue a step.
Constants come from one calibration workload and are then held fixed: the
device gap between dependent kernel launches, the same inside a graph, the
tile hand-off time, and the start of a persistent launch; an occupancy factor
for batched GEMVs comes from one batched workload.

Model.  One instruction of op o takes dur[o] = (K_o - R) / rounds_o, where
K_o is the op's per-op kernel time, R the time a launch of 256 near-empty
workgroups takes (the per-op embedding kernel, else the reset kernel), and
rounds_o = ceil(instructions / CUs).  Attention splits differ: split s of a
row with P keys reduces clamp(P - s kb, 0, kb) of them, so one takes
fixed + per_key * keys, with per_key such that the per-op launch (whose
workgroups the hardware hands out as CUs free up) takes the larger of its
longest split and its splits' total over the CUs.  An LM-head tile of a loop queue (no
per-op kernel of its own) runs the decode GEMV body: its time is read off a
straight line t0 + bytes / rate fitted to the GEMV ops' (weight bytes, dur)
pairs.  The tile pass, per instruction i in queue order on its worker:

    free  = end of the worker's previous instruction
    ready = max over waited barriers b of done[b] + hop     (free if none)
    lead  = min(prefetch[o], max(0, ready - free), dur[o])  (streamed while waiting)
    end   = max(free, ready) + dur[o] - lead
    done[signal] = max(done[signal], end)

Every waited barrier is signalled only by earlier instructions (queue order is
topological; the CPU checker verifies it) and a worker's previous instruction
is earlier too, so one pass in queue order gives every time.  A composition
of megakernels is the same pass with every worker held, at each cut, until
the previous launch's last instruction has ended, plus a launch gap, the
ramp of a new launch of 256 workgroups and the persistent launch's own start
beyond that ramp (a constant fitted on the calibration workload).  The
multi-stream pass is the same with each segment's instructions on the
8 * floor(CUs / 8 / S) workgroups of its own kernel, which starts when the
previous kernel of its stream (segment k - S) has ended.  A design's step is
max(device time, host enqueue time): the host enqueues c_call + c_launch per
launch, fitted to the measured enqueue times.

Host only; no device code.
"""
from __future__ import annotations

import json
import math
import re
import struct
from dataclasses import dataclass, field
from typing import Dict, List, Mapping, Optional, Sequence, Tuple

import numpy as np

OP_NAMES = {1: "EMBED", 2: "QKV", 3: "ATTN", 4: "COMBINE", 5: "OPROJ", 6: "GATEUP", 7: "DOWN",
            14: "LMHEAD", 15: "ARGMAX"}
OP_EMBED, OP_QKV, OP_ATTN, OP_COMBINE, OP_OPROJ, OP_GATEUP, OP_DOWN = 1, 2, 3, 4, 5, 6, 7
OP_LMHEAD, OP_ARGMAX = 14, 15
PREV = 0x80000000
LM_TILE = 64
XCDS = 8


@dataclass
class Graph:
    """The tile graph of a queue: per instruction op, layer, wait ranges and signal."""
    op: np.ndarray            # [n] int
    layer: np.ndarray         # [n] int
    wait_off: np.ndarray      # [n] first wait range
    wait_cnt: np.ndarray      # [n] number of wait ranges
    signal: np.ndarray        # [n] barrier signalled
    ranges: np.ndarray        # [n_ranges, 2] (first barrier, count with bit 31 = previous step)
    targets: np.ndarray       # [n_barriers]
    n_queues: int
    segments: List[Tuple[int, int, int, int]] = field(default_factory=list)   # (op, layer, first, count)
    flags: int = 0
    args: Optional[np.ndarray] = None    # [n, 3] the records' a0, a1, a2 (attention: row, KV head, split)


def graph_from_parts(parts: Mapping[str, bytes]) -> Graph:
    """Decode the META, INSTR, WAITS and TARGETS parts of an exported queue."""
    meta = parts["meta"]
    if meta[:4] != b"TMK1":
        raise ValueError("not a queue META part")
    h = struct.unpack_from("<20I", meta, 0)
    segs = [struct.unpack_from("<4I", meta, 80 + 16 * k) for k in range(h[6])]
    rec = np.frombuffer(parts["instr"], dtype="<u4").reshape(-1, 8)
    return Graph(op=(rec[:, 0] & 0xFFFF).astype(np.int64), layer=(rec[:, 0] >> 16).astype(np.int64),
                 wait_off=rec[:, 4].astype(np.int64), wait_cnt=rec[:, 5].astype(np.int64),
                 signal=rec[:, 6].astype(np.int64),
                 ranges=np.frombuffer(parts["waits"], dtype="<u4").reshape(-1, 2).astype(np.int64),
                 targets=np.frombuffer(parts["targets"], dtype="<u4").astype(np.int64),
                 n_queues=int(h[7]), segments=[tuple(int(v) for v in s) for s in segs], flags=int(h[19]),
                 args=rec[:, 1:4].astype(np.int64))


def _waits(g: Graph, i: int):
    """(same-step barrier runs, previous-step barrier runs) of instruction i."""
    same, prev = [], []
    for k in range(int(g.wait_off[i]), int(g.wait_off[i] + g.wait_cnt[i])):
        f, c = int(g.ranges[k, 0]), int(g.ranges[k, 1])
        (prev if c & PREV else same).append((f, c & ~PREV))
    return same, prev


def simulate(g: Graph, dur: Mapping[int, float], hop: float = 0.0,
             prefetch: Optional[Mapping[int, float]] = None,
             n_workers: Optional[int] = None, steps: int = 1,
             dur_i: Optional[np.ndarray] = None,
             pop_segments: Sequence[Tuple[int, int]] = (),
             cuts: Sequence[int] = (), cut_us: float = 0.0) -> Tuple[float, np.ndarray, np.ndarray]:
    """Event pass over the megakernel's schedule.  Returns (span, start, end) in
    the units of `dur`; start and end are those of the last step.  With as
    many workers as sub-queues (the default) position k of the repeated queue
    runs on worker k mod n_queues.  With more workers than sub-queues, the
    workers w, w + n_queues, ... share sub-queue w mod n_queues and pop from it
    in order: each instruction goes to the one of them that is free first.
    ``steps`` > 1 (loop queues): the queue repeated, a previous-step wait
    reading the previous step's barrier times.  ``dur_i`` (per instruction, NaN
    where the op's duration applies) overrides ``dur``.  ``pop_segments``
    (first, count): segments handed out at run time (one sub-queue per worker):
    the workers holding a position in the segment take its instructions in
    queue order, each going to the one of them that is free first.  ``cuts``
    (single step): positions where a new launch of a composition starts; no
    worker starts there or later before every earlier instruction has ended
    and ``cut_us`` more has passed."""
    nq = g.n_queues
    nw = n_workers or nq
    prefetch = prefetch or {}
    n = len(g.op)
    done_prev = np.zeros(len(g.targets))
    free = np.zeros(nw)
    members = [np.arange(q, nw, nq) for q in range(min(nq, nw))] if nw > nq else None
    waits = [_waits(g, i) for i in range(n)]
    start = np.zeros(n)
    end = np.zeros(n)
    pop_at = {f: c for f, c in pop_segments if c > 0}
    cut_at = set(int(c) for c in cuts if 0 < c < n)
    for t in range(steps):
        done = np.zeros(len(g.targets))
        i = 0
        while i < n:
            if i in cut_at:
                free[:] = free.max() + cut_us
            if i in pop_at and members is None:
                cnt = pop_at[i]
                part = np.unique((t * n + i + np.arange(min(cnt, nw))) % nw)
                for j in range(i, i + cnt):
                    w = int(part[np.argmin(free[part])])
                    f = free[w]
                    ready = f
                    for first, c in waits[j][0]:
                        ready = max(ready, float(done[first:first + c].max()) + hop)
                    op = int(g.op[j])
                    d = dur[op] if dur_i is None or np.isnan(dur_i[j]) else float(dur_i[j])
                    s = max(f, ready)
                    e = s + d
                    start[j], end[j] = s, e
                    free[w] = e
                    if e > done[g.signal[j]]:
                        done[g.signal[j]] = e
                i += cnt
                continue
            k = t * n + i
            if members is None:
                w = k % nw
            else:
                mq = members[k % nq]
                w = int(mq[np.argmin(free[mq])])
            f = free[w]
            ready = f
            same, prev = waits[i]
            for arr, runs in ((done, same), (done_prev, prev if t > 0 else [])):
                for first, cnt in runs:
                    ready = max(ready, float(arr[first:first + cnt].max()) + hop)
            op = int(g.op[i])
            d = dur[op] if dur_i is None or np.isnan(dur_i[i]) else float(dur_i[i])
            lead = min(prefetch.get(op, 0.0), max(0.0, ready - f), d)
            s = max(f, ready)
            e = s + d - lead
            start[i], end[i] = s, e
            free[w] = e
            sg = g.signal[i]
            if e > done[sg]:
                done[sg] = e
            i += 1
        done_prev = done
    return (float(free.max()) if n else 0.0), start, end


def layer_cuts(g: Graph, launches: int) -> List[int]:
    """Queue positions where launches 1..K-1 of a composition of K megakernels
    start: the first non-embedding instruction of layer k L / K."""
    n_layers = int(g.layer.max()) + 1 if len(g.layer) else 0
    first = {}
    for op, layer, f, _cnt in g.segments:
        if op != OP_EMBED:
            first[layer] = min(first.get(layer, f), f)
    return [first[k * n_layers // launches] for k in range(1, launches)]


def ms_grid(streams: int, n_cus: int, per_cu: int = 1) -> int:
    """Workgroups per kernel of the multi-stream mode (a multiple of the XCDs)."""
    return XCDS * ((per_cu * (n_cus // XCDS)) // streams)


def simulate_streams(g: Graph, dur: Mapping[int, float], hop: float, prefetch: Optional[Mapping[int, float]],
                     streams: int, n_cus: int, gap: float, dur_i: Optional[np.ndarray] = None) -> float:
    """Multi-stream mode: segment k is a kernel on stream k mod S with its own
    ms_grid(S) workgroups striding over its instructions; it starts `gap`
    after the previous kernel of its stream ends.  Returns the span."""
    prefetch = prefetch or {}
    G = ms_grid(streams, n_cus)
    done = np.zeros(len(g.targets))
    sfree = [0.0] * streams
    for k, (op, _layer, first, count) in enumerate(g.segments):
        s = k % streams
        kstart = sfree[s] + gap
        wfree = [kstart] * min(G, count)
        kend = kstart
        for j in range(count):
            i = first + j
            w = j % G
            f = wfree[w]
            ready = f
            for a, c in _waits(g, i)[0]:
                ready = max(ready, float(done[a:a + c].max()) + hop)
            d = dur[int(g.op[i])] if dur_i is None or np.isnan(dur_i[i]) else float(dur_i[i])
            lead = min(prefetch.get(int(g.op[i]), 0.0), max(0.0, ready - f), d)
            e = max(f, ready) + d - lead
            wfree[w] = e
            done[g.signal[i]] = max(done[g.signal[i]], e)
            kend = max(kend, e)
        sfree[s] = kend
    return max(sfree)


def op_counts(g: Graph) -> Dict[int, int]:
    """Instructions per op in one (layer, op) segment (the op's per-op launch size)."""
    out: Dict[int, int] = {}
    for op, _layer, _first, count in g.segments:
        out[op] = max(out.get(op, 0), count)
    return out


def per_instruction_us(kernel_us: Mapping[int, float], counts: Mapping[int, int], n_cus: int,
                       ramp_us: float = 0.0) -> Dict[int, float]:
    """One instruction's run time from a per-op kernel's time: a launch of n
    instructions pays the launch ramp once, then runs ceil(n / n_cus) rounds
    of concurrent workgroups."""
    return {op: max(kernel_us[op] - ramp_us, 0.05 * kernel_us[op]) / max(1, -(-counts[op] // n_cus))
            for op in kernel_us if op in counts}


# Fixed part of an attention split (µs): reading q, k, v and rotating them after
# its wait, merging the lane groups' and waves' softmax states, storing the
# partial and signalling; from the batch-1 trace of the 8B step (1.5 + 3 µs).
ATTN_FIXED_US = 4.5


def split_keys(g: Graph, ctx: Sequence[int], kb: int) -> np.ndarray:
    """Keys each attention instruction reduces (NaN for other ops): the split s
    of row b covers keys [s kb, (s + 1) kb) of the row's ctx[b] (cache plus the
    new token)."""
    out = np.full(len(g.op), np.nan)
    if g.args is None:
        return out
    at = g.op == OP_ATTN
    b, s = g.args[at, 0], g.args[at, 2]
    c = np.asarray(ctx, dtype=np.float64)[b]
    out[at] = np.clip(c - s * kb, 0, kb)
    return out


def attention_durations(kernel_us: float, ramp_us: float, keys: np.ndarray, n_layers_ops: int, n_cus: int,
                        fixed_us: float = ATTN_FIXED_US) -> np.ndarray:
    """Per-instruction attention times fixed + per_key * keys (NaN elsewhere).
    The per-op launch of one layer's splits hands workgroups out as CUs free
    up, so its net time is the larger of its longest split and its splits' total
    over the CUs; per_key is the value that makes that equal the measured kernel
    time.  ``n_layers_ops``: the number of attention launches the instructions
    span (one per layer)."""
    out = np.full(len(keys), np.nan)
    at = ~np.isnan(keys)
    if not at.any():
        return out
    net = max(kernel_us - ramp_us, 0.05 * kernel_us)
    k = keys[at]
    n = k.size / max(1, n_layers_ops)                   # splits per launch
    ksum = k.sum() / max(1, n_layers_ops)
    kmax = float(k.max())
    fixed = min(fixed_us, 0.9 * net)
    p_one = (net - fixed) / kmax if kmax > 0 else np.inf        # bound by the longest split
    p_all = (net * n_cus - fixed * n) / ksum if ksum > 0 else np.inf   # bound by the total
    per_key = max(0.0, min(p_one, p_all))
    out[at] = fixed + per_key * k
    return out


def kpo_step(g: Graph, kernel_us: Mapping[int, float], gap_us: float) -> float:
    """Kernel-per-op layers: every (layer, op) launch in turn, plus a launch gap each."""
    return sum(kernel_us[op] for op, *_ in g.segments) + len(g.segments) * gap_us


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


@dataclass
class Timings:
    """Standalone kernel times of one workload, µs."""
    kernel_us: Dict[int, float]
    lm_us: float = 0.0
    argmax_us: float = 0.0
    reset_us: float = 0.0
    copy_us: float = 0.0
    ramp_us: float = 0.0          # a launch of 256 near-empty workgroups

    @staticmethod
    def from_rows(rows: Sequence[Tuple[str, float]]) -> "Timings":
        def avg(key):
            v = [ns / 1000.0 for n, ns in rows if key in n]
            return v[0] if v else 0.0
        k = kpo_kernel_us(rows)
        t = Timings(k, lm_us=avg("lm_head_"), argmax_us=avg("argmax_kernel"), reset_us=avg("reset_kernel"),
                    copy_us=avg("copy_rows_kernel"))
        t.ramp_us = k.get(OP_EMBED, t.reset_us)
        return t


def gemv_line(dur: Mapping[int, float], weight_bytes: Mapping[int, int]) -> Tuple[float, float]:
    """Least-squares line dur = t0 + bytes / rate over the GEMV ops; (t0 µs, rate bytes/µs)."""
    pts = [(weight_bytes[o], dur[o]) for o in (OP_QKV, OP_OPROJ, OP_GATEUP, OP_DOWN) if o in dur and o in weight_bytes]
    x = np.array([p[0] for p in pts], dtype=np.float64)
    y = np.array([p[1] for p in pts], dtype=np.float64)
    slope, t0 = np.polyfit(x, y, 1)
    return float(max(t0, 0.0)), float(1.0 / max(slope, 1e-12))


def gemv_prefetch_us(dur: Mapping[int, float], weight_bytes: Mapping[int, int], ring_bytes: int) -> Dict[int, float]:
    """Time's worth of a GEMV instruction's weights that its ring holds before it
    waits: the ring's share of the instruction's weight bytes, times its run time."""
    return {op: min(1.0, ring_bytes / b) * dur[op] for op, b in weight_bytes.items() if op in dur}


@dataclass
class Calib:
    """Constants fitted on calibration workloads (µs, or a factor)."""
    gap_us: float = 0.3           # device gap between dependent launches, eager
    graph_gap_us: float = 0.3     # the same inside a replayed graph
    hop_us: float = 1.0           # tile hand-off: producer's signal to consumer running
    mega_launch_us: float = 0.0   # a megakernel launch's start beyond a near-empty launch's ramp
    occupancy: float = 1.0        # batched GEMV instruction in the interpreter / in its per-op kernel
    host_call_us: float = 30.0    # host: enqueueing a step, fixed part
    host_launch_us: float = 2.0   # host: per kernel launch
    graph_call_us: float = 50.0   # host: a graph replay, fixed part
    graph_node_us: float = 0.1    # host: per kernel node of the replayed graph


@dataclass
class Workload:
    """What the predictor needs of one workload."""
    name: str
    single: Graph                 # the step's queue
    loop: Optional[Graph]         # its loop queue (LM head inside), if the model has one
    timings: Timings
    weight_bytes: Dict[int, int]  # weight bytes of one instruction per GEMV op (and the LM-head tile)
    ring_bytes: int
    rows: int
    has_lm: bool
    has_embed: bool
    n_cus: int = 256
    ctx: Optional[Sequence[int]] = None   # keys each row's attention covers (cache plus the new token)
    kb: int = 0                           # keys per attention split
    attn_pop: bool = False                # the megakernel hands the splits out at run time


def _launches(w: Workload, design: str) -> float:
    """Kernel launches the host enqueues per step."""
    pre = 0 if w.has_embed else 1                       # input-row copy
    lm = 2 if w.has_lm else 0
    if design == "mega":
        return pre + 2 + lm
    if design.startswith("mega"):
        return pre + 1 + int(design[4:]) + lm
    if design in ("kpo", "kpo_graph"):
        return pre + 1 + len(w.single.segments) + lm          # kernels (graph nodes)
    if design == "loop":
        return 0.0
    if design.startswith("ms"):
        s = int(design[2:])
        return pre + 1 + len(w.single.segments) + 2 * s + 1 + lm
    raise ValueError(design)


def predict(w: Workload, c: Calib, designs: Sequence[str] = ("mega", "kpo", "kpo_graph", "loop", "ms2", "ms4",
                                                              "mega2", "mega3", "mega4"),
            loop_steps: int = 32, host_us: Optional[Mapping[str, Optional[float]]] = None
            ) -> Dict[str, Dict[str, float]]:
    """Predicted device, host and step times (µs) of each design.  ``host_us``:
    the workload's own measured host enqueue time per design, where there is
    one (measured on the host alone); else the fitted host lines."""
    t = w.timings
    dur = per_instruction_us(t.kernel_us, op_counts(w.single), w.n_cus, t.ramp_us)
    # the interpreter runs one wave per SIMD; a batched GEMV's per-op kernel runs
    # several and hides more of its arithmetic latency
    occ = c.occupancy if w.rows > 2 else 1.0
    dur_mk = {o: v * (occ if o in (OP_QKV, OP_OPROJ, OP_GATEUP, OP_DOWN) else 1.0) for o, v in dur.items()}
    pre = 0.0 if w.has_embed else t.copy_us
    lm = (t.lm_us + t.argmax_us + 2 * c.gap_us) if w.has_lm else 0.0
    pf = gemv_prefetch_us(dur_mk, w.weight_bytes, w.ring_bytes)

    def attn_i(g: Graph) -> Optional[np.ndarray]:
        # attention splits weighted by their keys (ragged contexts load workers unevenly)
        if w.ctx is None or not w.kb or OP_ATTN not in t.kernel_us:
            return None
        n_launch = sum(1 for op, *_ in g.segments if op == OP_ATTN) or 1
        return attention_durations(t.kernel_us[OP_ATTN], t.ramp_us, split_keys(g, w.ctx, w.kb), n_launch,
                                   w.n_cus)
    ai = attn_i(w.single)
    out: Dict[str, Dict[str, float]] = {}
    for d in designs:
        if d.startswith("mega"):
            pops = [(f, cnt) for op, _l, f, cnt in w.single.segments if op == OP_ATTN] \
                if w.attn_pop and w.single.n_queues >= w.n_cus else []
            k = 1 if d == "mega" else int(d[4:])
            if k > 1 and (w.single.n_queues != w.n_cus or k > int(w.single.layer.max()) + 1):
                continue                                # the library refuses it
            cuts = layer_cuts(w.single, k) if k > 1 else []
            span, _, _ = simulate(w.single, dur_mk, c.hop_us, pf,
                                  n_workers=w.n_cus if w.single.n_queues < w.n_cus else None, dur_i=ai,
                                  pop_segments=pops, cuts=cuts,
                                  cut_us=c.gap_us + t.ramp_us + c.mega_launch_us)
            # the launch of 256 persistent workgroups costs what a near-empty launch does
            dev = pre + t.reset_us + t.ramp_us + span + lm + 2 * c.gap_us
        elif d in ("kpo", "kpo_graph"):
            gap = c.gap_us if d == "kpo" else c.graph_gap_us
            lm_d = (t.lm_us + t.argmax_us + 2 * gap) if w.has_lm else 0.0
            dev = pre + t.reset_us + kpo_step(w.single, t.kernel_us, gap) + lm_d + gap
        elif d == "loop":
            if w.loop is None or not w.has_lm:
                continue
            d2 = dict(dur_mk)
            t0, rate = gemv_line(dur, w.weight_bytes)
            d2[OP_LMHEAD] = (t0 + w.weight_bytes.get(OP_LMHEAD, 0) / rate) * occ
            d2[OP_ARGMAX] = t.argmax_us
            pf2 = gemv_prefetch_us(d2, w.weight_bytes, w.ring_bytes)
            nw = w.n_cus if w.loop.n_queues < w.n_cus else None
            li = attn_i(w.loop)
            s1, _, _ = simulate(w.loop, d2, c.hop_us, pf2, n_workers=nw, steps=1, dur_i=li)
            s2, _, _ = simulate(w.loop, d2, c.hop_us, pf2, n_workers=nw, steps=2, dur_i=li)
            per_step = s2 - s1
            dev = per_step + (t.reset_us + t.ramp_us + s1 - per_step) / loop_steps
        elif d.startswith("ms"):
            # per-op kernels again (their occupancy), each paying its own launch
            span = simulate_streams(w.single, dur, c.hop_us, gemv_prefetch_us(dur, w.weight_bytes, w.ring_bytes),
                                    int(d[2:]), w.n_cus, c.gap_us + t.ramp_us, dur_i=ai)
            dev = pre + t.reset_us + span + lm + 2 * c.gap_us
        else:
            raise ValueError(d)
        if host_us and host_us.get(d) is not None:
            host = float(host_us[d])
        elif d == "loop":
            host = c.host_call_us / loop_steps
        elif d == "kpo_graph":
            host = c.graph_call_us + c.graph_node_us * _launches(w, d)
        else:
            host = c.host_call_us + c.host_launch_us * _launches(w, d)
        out[d] = {"device_us": dev, "host_us": host, "step_us": max(dev, host)}
    return out


def _fit(f, lo: float, hi: float, target: float) -> float:
    """x in [lo, hi] with f(x) = target for an increasing f (bisection)."""
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if f(mid) < target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def calibrate(w: Workload, measured_us: Mapping[str, float],
              host_enqueue_us: Sequence[Tuple[Workload, str, float]] = (),
              batched: Optional[Tuple[Workload, float]] = None, base: Optional[Calib] = None) -> Calib:
    """Fit the constants: the launch gaps and the hand-off time on workload
    ``w``'s measured steps (batch 1), the occupancy factor on a batched
    workload's measured megakernel step, and the host line over every
    (workload, design, enqueue µs) given, from GPU-bound workloads."""
    c = Calib(**(base.__dict__ if base else {}))
    t = w.timings
    pre = 0.0 if w.has_embed else t.copy_us
    lm_k = (t.lm_us + t.argmax_us) if w.has_lm else 0.0
    n_lm = 2 if w.has_lm else 0
    ksum = sum(t.kernel_us[op] for op, *_ in w.single.segments)
    n_seg = len(w.single.segments)
    c.gap_us = max(0.0, (measured_us["kpo"] - pre - t.reset_us - ksum - lm_k) / (n_seg + 1 + n_lm))
    c.graph_gap_us = max(0.0, (measured_us["kpo_graph"] - pre - t.reset_us - ksum - lm_k) / (n_seg + 1 + n_lm))
    def with_(**kw):
        return Calib(**{**c.__dict__, **kw})
    c.hop_us = _fit(lambda h: predict(w, with_(hop_us=h), ("mega",))["mega"]["device_us"], 0.0, 50.0,
                    measured_us["mega"])
    if "mega2" in measured_us:
        # what a cut costs beyond the drain, the gap and a near-empty launch: the
        # persistent launch's own start (the library refuses compositions of
        # shared sub-queues, so a plan with them has no mega2)
        c.mega_launch_us = _fit(lambda x: predict(w, with_(mega_launch_us=x), ("mega2",))["mega2"]["device_us"],
                                0.0, 100.0, measured_us["mega2"])
    if batched is not None:
        wb, mega_b = batched
        c.occupancy = _fit(lambda f: predict(wb, with_(occupancy=f), ("mega",))["mega"]["device_us"], 0.5, 4.0,
                           mega_b)
    for graph in (False, True):
        pts = [(_launches(wl, d), us) for wl, d, us in host_enqueue_us if (d == "kpo_graph") == graph]
        if len({x for x, _ in pts}) >= 2:
            slope, icpt = np.polyfit(np.array([x for x, _ in pts], dtype=np.float64),
                                     np.array([y for _, y in pts], dtype=np.float64), 1)
            if graph:
                c.graph_node_us, c.graph_call_us = float(max(slope, 0.0)), float(max(icpt, 0.0))
            else:
                c.host_launch_us, c.host_call_us = float(max(slope, 0.0)), float(max(icpt, 0.0))
    return c


def co_best(times: Mapping[str, float], tol: float = 0.01) -> List[str]:
    """The designs within `tol` of the fastest (measurements closer than that
    are not told apart)."""
    b = min(times.values())
    return sorted(d for d, v in times.items() if v <= b * (1 + tol))


def best(times: Mapping[str, float]) -> str:
    return min(times, key=times.get)


# ----------------------------------------------------------------------------- workloads from the library

def workload(name: str, stats_rows: Sequence[Tuple[str, float]], n_cus: int = 256) -> Workload:
    """Build the queues of a benchmark workload with the library and read its
    standalone kernel times."""
    import dataclasses
    import tile_synchronized_decoder_amd as T
    import workloads as W
    wl = W.WORKLOADS[name]
    m, r, p = wl.model, wl.run, wl.plan
    q = T.mk_build_queue(T.make_config(m), T.make_plan(p, T.MK_DECODE, r.batch, r.ctx_max))
    single = graph_from_parts(q.parts())
    loop = None
    if m.has_embed and m.has_lm_head and m.dtype == "bf16":
        ql = T.mk_build_queue(T.make_config(m), T.make_plan(dataclasses.replace(p, loop=1, attn_pop=0), T.MK_DECODE,
                                                            r.batch, r.ctx_max))
        loop = graph_from_parts(ql.parts())
    es = 2 if m.dtype == "bf16" else 4
    na = m.n_q_heads * m.head_dim
    wbytes = {OP_QKV: p.tq * m.hidden * es, OP_OPROJ: p.to * na * es, OP_GATEUP: 2 * p.tf * m.hidden * es,
              OP_DOWN: p.td * m.ffn * es, OP_LMHEAD: LM_TILE * m.hidden * es}
    ring = 4 * (20 if r.batch <= 2 else 16) * 1024          # four waves' weight rings (1 KB lines)
    ctx = [c0 + 1 for c0 in r.ctx0]                        # the first timed step's keys per row
    return Workload(name, single, loop, Timings.from_rows(stats_rows), wbytes, ring, r.batch,
                    m.has_lm_head, m.has_embed, n_cus, ctx=ctx, kb=p.kb, attn_pop=bool(getattr(p, "attn_pop", 0)))


def read_mode_times(path: str) -> Dict[str, Dict[str, Dict[str, float]]]:
    """Measured step times and host enqueue times, workload -> design -> {step_us, host_us},
    from the JSON lines after the `measured:` marker of a predictor summary."""
    out: Dict[str, Dict[str, Dict[str, float]]] = {}
    on = False
    with open(path) as f:
        for line in f:
            if line.startswith("<!-- measured"):
                on = True
                continue
            if on and line.startswith("-->"):
                break
            if on and line.strip():
                rec = json.loads(line)
                out.setdefault(rec["workload"], {})[rec["design"]] = {"step_us": rec["step_us"],
                                                                      "host_us": rec.get("host_us")}
    return out


def check(names: Sequence[str], profiles_dir: str, calib_on: str = "llama1b_b1",
          calib_batched: str = "llama8b_b16") -> Dict[str, dict]:
    """Predict every design of every workload from its kernel summary
    (profiles/mk_interp_<name>_kernels.md), calibrating on one of them, and
    compare with the measured times in profiles/predictor_check.md."""
    import os
    meas = read_mode_times(os.path.join(profiles_dir, "predictor_check.md"))
    wls = {n: workload(n, read_kernel_stats_md(os.path.join(profiles_dir, f"mk_interp_{n}_kernels.md")))
           for n in names}
    # host enqueue times of GPU-bound workloads (steps far longer than enqueueing them)
    host = [(wls[n], d, v["host_us"]) for n in names if n in meas and meas[n].get("mega", {}).get("step_us", 0) > 500
            for d, v in meas[n].items() if v.get("host_us") and d in ("mega", "kpo", "kpo_graph", "ms2", "ms4",
                                                                       "mega2", "mega3", "mega4")]
    bat = (wls[calib_batched], meas[calib_batched]["mega"]["step_us"]) if calib_batched in wls else None
    c = calibrate(wls[calib_on], {d: v["step_us"] for d, v in meas[calib_on].items()}, host, bat)
    res = {"calibration": {"workloads": [calib_on, calib_batched],
                           **{k: round(v, 3) for k, v in c.__dict__.items()}}}
    for n in names:
        pred = predict(wls[n], c, host_us={d: v.get("host_us") for d, v in meas.get(n, {}).items()})
        m = {d: v["step_us"] for d, v in meas.get(n, {}).items() if d in pred}
        p = {d: v["step_us"] for d, v in pred.items()}
        entry = {"predicted_us": {d: round(v, 1) for d, v in p.items()},
                 "measured_us": {d: round(v, 1) for d, v in m.items()},
                 "error_pct": {d: round(100 * (p[d] / m[d] - 1), 1) for d in m},
                 "pick": best({d: p[d] for d in m}), "measured_best": co_best(m) if m else []}
        entry["pick_ok"] = entry["pick"] in entry["measured_best"]
        if "loop" in p and "mega" in p:
            entry["lm_head"] = "inside" if p["loop"] < p["mega"] else "separate"
            if "loop" in m and "mega" in m:
                # within co_best's 1% the two placements are not told apart
                tie = set(co_best({"loop": m["loop"], "mega": m["mega"]})) == {"loop", "mega"}
                entry["measured_lm_head"] = "either" if tie else "inside" if m["loop"] < m["mega"] else "separate"
        res[n] = entry
    return res


def main():
    import argparse
    import os
    ap = argparse.ArgumentParser(description="predict the decode designs' step times from standalone kernel "
                                             "timings and compare with measurement")
    ap.add_argument("--profiles", default=os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                                       "profiles"))
    ap.add_argument("--workloads", default="layer256_f32,llama1b_b1,llama8b_b1,llama8b_b4,llama8b_b16,"
                                           "llama1b_stream_b32,qwen8b_prefill")
    ap.add_argument("--calibrate-on", default="llama1b_b1")
    a = ap.parse_args()
    print(json.dumps(check(a.workloads.split(","), a.profiles, a.calibrate_on), indent=1))


if __name__ == "__main__":
    main()
