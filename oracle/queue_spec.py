"""Reference builder of the instruction queue and its tile barriers (test infrastructure).

What the pages fix: the decoder runs as an interpreter that pops instructions
from one queue in device memory ("Production Megakernels" lecture summary,
Technical details: execution model); the queue is built once with sequence and
context lengths kept symbolic (Key takeaways: symbolic representation of work);
barriers are tensors whose dimensions are partitioned by dependency (Key
takeaways: dependency tracking); a consumer waits on the tiles of the
intermediate tensor it reads, not on whole kernels (MegaOps abstract).

What the pages leave open and this module fixes (the plainest reading):

* Every instruction writes exactly one tile of one intermediate tensor and
  reads a list of rectangular regions.  Intermediates are distinct per layer,
  so only read-after-write dependencies exist.
* One barrier counter per written tile; its target is the number of
  instructions that write that tile.  Barrier ids are numbered in order of the
  tile's first write in queue order.
* The wait list of an instruction is every written tile whose box intersects
  one of its read regions (plain box intersection), ordered by (tensor order,
  column start, row start).  It is stored as ranges: maximal runs of that
  ordered list whose barrier ids are consecutive become one (first, count).
* Queue order is canonical: embedding tiles, then per layer the QKV tiles, the
  attention splits (split-major: for split s, the (row, KV head) pairs in
  order starting s rows on, cyclically, so that the instructions a worker
  takes by position span several rows), the split combines (KV head, row) --
  the order in which their output tiles lie along the columns, so a reader of
  the whole attention output waits on one run of consecutive barriers -- then
  the O-projection, gate/up and down tiles (decode); the prefill queue has the same shape over 2-D row x column
  tiles.  The context length only enters through NS = ceil(ctx_max / KB)
  splits, so the queue is independent of the runtime context (and of the
  runtime prompt length in prefill, whose unused row blocks become no-ops).
* With the plan's ``fuse_combine`` set to 1 (decode), the split combines are
  not instructions of their own: each O-projection tile reads the split
  partials of every (row, KV head) in place of the attention output and
  merges them while staging its inputs; the attention-output tensor then has
  no tiles.  Bit 0 of the META word after bn records it.
* With ``fuse_combine`` 2 the queue has the same instructions and wait lists
  as with 1, and the O-projection tiles still wait on the partial tiles, but
  the merge happens at the end of the attention: every split counts its
  arrival on its (row, KV head) partial tile, and the split whose arrival
  brings the count to NS merges the NS partials into that row's attention
  output (the attention-output tensor, as with the combines) and signals the
  tile once more.  The partial tile's target is therefore NS + 1; the
  O-projection tiles read the merged attention output.  Bit 2 of the META
  word records it.
* With the plan's ``loop`` set (decode, persistent multi-step decode; the
  lecture summary's practical implications keep the host out of the hot
  loop), one queue describes one step of a run of T steps that one launch
  executes in order.  After the layers come the LM-head tiles LMHEAD(v0, v1)
  (64 vocabulary rows each, reading all of X_L and writing that tile of the
  logits) and one ARGMAX(b) per row (reading its whole logits row and writing
  the row's next token).  Every EMBED tile reads the next-token tensor of the
  previous step: those waits form ranges of their own, after the same-step
  ones, marked by bit 31 of the range count (PREV).  At step t a worker waits
  until a same-step barrier's counter reaches target * (t + 1), a
  previous-step one until target * t, so the counters are cleared once per
  launch.  Buffers are reused across steps; that is safe because every
  instruction of a step is an ancestor of some ARGMAX and every instruction
  descends from some EMBED tile, which waits for all of the previous step's
  ARGMAX (the checker verifies both).  The META flags word gets bit 1.

Byte layout (little-endian), shared with the GPU library's C builder:

META    u32 magic 'TMK1', version, mode, n_instr, n_barriers, n_wait_ranges, n_segments,
        n_queues, rows, ctx_max, n_splits, n_layers, tq, to, tf, td, kb, bm, bn, flags
        (bit 0: split combines fused into the O-projection; bit 1: multi-step loop queue;
        bit 2: split combines merged by the last-arriving split; bit 3: attention
        splits handed out at run time, same instructions),
        then n_segments x {u32 op, layer, first, count} (maximal runs of one op of one layer)
INSTR   n_instr x 32 B {u16 op, u16 layer, u32 a0, a1, a2, wait_off, wait_cnt, signal, n_wait}
        (wait_off/wait_cnt index WAITS ranges; n_wait = barriers waited on in total)
WAITS   n_wait_ranges x {u32 first barrier id, u32 count} (count bit 31: previous-step barriers)
TARGETS n_barriers x u32 (signalling instructions; + 1 for a partial tile under bit 2)
"""
from __future__ import annotations

import math
import struct
from dataclasses import dataclass, field
from typing import Dict, List, Tuple

MAGIC = 0x314B4D54          # b"TMK1" little-endian
VERSION = 1
MODE_DECODE, MODE_PREFILL = 0, 1

OP_EMBED, OP_QKV, OP_ATTN, OP_COMBINE, OP_OPROJ, OP_GATEUP, OP_DOWN = 1, 2, 3, 4, 5, 6, 7
OP_P_EMBED, OP_P_QKV, OP_P_ATTN, OP_P_OPROJ, OP_P_GATEUP, OP_P_DOWN = 8, 9, 10, 11, 12, 13
OP_LMHEAD, OP_ARGMAX = 14, 15
OP_NAMES = {1: "EMBED", 2: "QKV", 3: "ATTN", 4: "COMBINE", 5: "OPROJ", 6: "GATEUP", 7: "DOWN",
            8: "P_EMBED", 9: "P_QKV", 10: "P_ATTN", 11: "P_OPROJ", 12: "P_GATEUP", 13: "P_DOWN",
            14: "LMHEAD", 15: "ARGMAX"}
LM_TILE = 64                  # vocabulary rows per LM-head tile of a loop queue
PREV = 0x80000000             # range-count flag: barriers of the previous step

# tensor kinds within a layer, in tensor order
T_QKV, T_OPART, T_ATT, T_HRES, T_ACT, T_XNEXT = range(6)
MAX_DECODE_ROWS = 32
MAX_QUEUES = 1024


class QueueError(ValueError):
    pass


def tensor_order(layer: int, kind: int) -> int:
    """Global tensor index: X_0 is 0, then six tensors per layer (X_{l+1} last)."""
    return 1 + 6 * layer + kind


def x_tensor(layer: int) -> int:
    """Tensor index of X_layer (the input rows of ``layer``)."""
    return 0 if layer == 0 else tensor_order(layer - 1, T_XNEXT)


def logits_tensor(n_layers: int) -> int:
    """Tensor index of the logits [rows, V] of a loop queue (after the layers)."""
    return 1 + 6 * n_layers


def next_tensor(n_layers: int) -> int:
    """Tensor index of the next tokens [rows, 1] of a loop queue."""
    return 2 + 6 * n_layers


Box = Tuple[int, int, int, int]        # row0, row1, col0, col1 (half-open)


@dataclass
class Instr:
    op: int
    layer: int
    a0: int
    a1: int
    a2: int
    write: Tuple[int, Box]
    reads: List[Tuple[int, Box]]
    prev_reads: List[Tuple[int, Box]] = field(default_factory=list)   # the previous step's tiles
    wait_off: int = 0
    wait_cnt: int = 0
    signal: int = 0
    n_wait: int = 0


@dataclass
class Queue:
    mode: int
    rows: int
    ctx_max: int
    n_splits: int
    n_layers: int
    plan: Tuple[int, ...]              # tq, to, tf, td, kb, bm, bn
    n_queues: int
    flags: int = 0
    instrs: List[Instr] = field(default_factory=list)
    waits: List[Tuple[int, int]] = field(default_factory=list)      # (first, count) ranges
    targets: List[int] = field(default_factory=list)
    tiles: List[Tuple[int, Box]] = field(default_factory=list)   # barrier id -> (tensor, box)
    segments: List[Tuple[int, int, int, int]] = field(default_factory=list)

    # -- serialisation
    def meta_bytes(self) -> bytes:
        head = struct.pack("<20I", MAGIC, VERSION, self.mode, len(self.instrs), len(self.targets),
                           len(self.waits), len(self.segments), self.n_queues, self.rows,
                           self.ctx_max, self.n_splits, self.n_layers, *self.plan, self.flags)
        return head + b"".join(struct.pack("<4I", *s) for s in self.segments)

    def instr_bytes(self) -> bytes:
        return b"".join(struct.pack("<HH7I", i.op, i.layer, i.a0, i.a1, i.a2, i.wait_off,
                                    i.wait_cnt, i.signal, i.n_wait) for i in self.instrs)

    def waits_bytes(self) -> bytes:
        return b"".join(struct.pack("<2I", f, c) for f, c in self.waits)

    def wait_list(self, i: int, prev: bool = False) -> List[int]:
        """Expanded barrier ids instruction i waits on in its own step (or, with
        ``prev``, in the previous step), in wait-list order."""
        ins = self.instrs[i]
        out: List[int] = []
        for f, c in self.waits[ins.wait_off: ins.wait_off + ins.wait_cnt]:
            if bool(c & PREV) == prev:
                out.extend(range(f, f + (c & ~PREV)))
        return out

    def targets_bytes(self) -> bytes:
        return struct.pack(f"<{len(self.targets)}I", *self.targets)

    def parts(self) -> Dict[str, bytes]:
        return {"meta": self.meta_bytes(), "instr": self.instr_bytes(),
                "waits": self.waits_bytes(), "targets": self.targets_bytes()}


def _tiles(n: int, t: int) -> List[Tuple[int, int]]:
    """Column (or row) tiles of width t over [0, n); the last one holds the remainder."""
    return [(s, min(s + t, n)) for s in range(0, n, t)]


def _overlap(a: Box, b: Box) -> bool:
    return a[0] < b[1] and b[0] < a[1] and a[2] < b[3] and b[2] < a[3]


def _check(model, plan, mode: int, rows: int, ctx_max: int) -> None:
    dims = (model.n_layers, model.hidden, model.n_q_heads, model.n_kv_heads, model.head_dim,
            model.ffn)
    if any(d <= 0 for d in dims):
        raise QueueError("model dimensions must be positive")
    if model.n_q_heads % model.n_kv_heads:
        raise QueueError("query heads must be a multiple of KV heads")
    if model.head_dim % 2:
        raise QueueError("head_dim must be even (rotary pairs)")
    if model.has_embed and model.vocab <= 0:
        raise QueueError("an embedding needs a vocabulary")
    if rows <= 0 or ctx_max <= 0:
        raise QueueError("rows and ctx_max must be positive")
    if not 1 <= plan.n_queues <= MAX_QUEUES:
        raise QueueError("n_queues out of range")
    if getattr(plan, "fuse_combine", 0) not in (0, 1, 2):
        raise QueueError("fuse_combine must be 0, 1 or 2")
    if getattr(plan, "loop", 0) not in (0, 1):
        raise QueueError("loop must be 0 or 1")
    if getattr(plan, "loop", 0) and (mode != MODE_DECODE or not model.has_embed or not model.has_lm_head):
        raise QueueError("a loop queue decodes a model with an embedding and an LM head")
    if getattr(plan, "attn_pop", 0) not in (0, 1):
        raise QueueError("attn_pop must be 0 or 1")
    if getattr(plan, "attn_pop", 0) and (mode != MODE_DECODE or getattr(plan, "loop", 0)):
        raise QueueError("attn_pop is for single-step decode queues")
    if mode == MODE_DECODE:
        if rows > MAX_DECODE_ROWS:
            raise QueueError("decode rows above the maximum")
        if min(plan.tq, plan.to, plan.tf, plan.td, plan.kb) <= 0:
            raise QueueError("tile sizes must be positive")
    elif mode == MODE_PREFILL:
        if min(plan.bm, plan.bn) <= 0:
            raise QueueError("tile sizes must be positive")
        if plan.bn % model.head_dim:
            raise QueueError("prefill column tile must hold whole heads")
        if rows > ctx_max:
            raise QueueError("prefill rows exceed the cache")
    else:
        raise QueueError("unknown mode")


def _decode_instrs(model, plan, M: int, NS: int) -> List[Instr]:
    H, F, hd = model.hidden, model.ffn, model.head_dim
    nq, nkv, r = model.n_q_heads, model.n_kv_heads, model.group
    NQKV, NA = model.qkv_cols, model.attn_cols
    out: List[Instr] = []
    loop = getattr(plan, "loop", 0)
    NEXT, LOGITS = next_tensor(model.n_layers), logits_tensor(model.n_layers)
    if model.has_embed:
        for n0, n1 in _tiles(H, plan.td):
            out.append(Instr(OP_EMBED, 0, n0, n1, 0, (0, (0, M, n0, n1)), [],
                             [(NEXT, (0, M, 0, 1))] if loop else []))
    for l in range(model.n_layers):
        X = x_tensor(l)
        QKV, OP, ATT = tensor_order(l, T_QKV), tensor_order(l, T_OPART), tensor_order(l, T_ATT)
        HR, ACT, XN = tensor_order(l, T_HRES), tensor_order(l, T_ACT), tensor_order(l, T_XNEXT)
        for n0, n1 in _tiles(NQKV, plan.tq):
            out.append(Instr(OP_QKV, l, n0, n1, 0, (QKV, (0, M, n0, n1)), [(X, (0, M, 0, H))]))
        # split-major; the (row, KV head) pairs are rotated by one row per split
        P = M * nkv
        for s in range(NS):
            for t in range(P):
                b, g = divmod((t + s * nkv) % P, nkv)
                qc = (g * r * hd, (g + 1) * r * hd)
                kc = (nq * hd + g * hd, nq * hd + (g + 1) * hd)
                vc = ((nq + nkv) * hd + g * hd, (nq + nkv) * hd + (g + 1) * hd)
                out.append(Instr(OP_ATTN, l, b, g, s, (OP, (b, b + 1, g, g + 1)),
                                 [(QKV, (b, b + 1) + qc), (QKV, (b, b + 1) + kc),
                                  (QKV, (b, b + 1) + vc)]))
        fused = getattr(plan, "fuse_combine", 0)
        if not fused:
            for g in range(nkv):
                for b in range(M):
                    out.append(Instr(OP_COMBINE, l, b, g, 0, (ATT, (b, b + 1, g * r * hd, (g + 1) * r * hd)),
                                     [(OP, (b, b + 1, g, g + 1))]))
        att_read = (OP, (0, M, 0, nkv)) if fused else (ATT, (0, M, 0, NA))
        for n0, n1 in _tiles(H, plan.to):
            out.append(Instr(OP_OPROJ, l, n0, n1, 0, (HR, (0, M, n0, n1)),
                             [att_read, (X, (0, M, n0, n1))]))
        for n0, n1 in _tiles(F, plan.tf):
            out.append(Instr(OP_GATEUP, l, n0, n1, 0, (ACT, (0, M, n0, n1)), [(HR, (0, M, 0, H))]))
        for n0, n1 in _tiles(H, plan.td):
            out.append(Instr(OP_DOWN, l, n0, n1, 0, (XN, (0, M, n0, n1)),
                             [(ACT, (0, M, 0, F)), (HR, (0, M, n0, n1))]))
    if loop:
        XL = x_tensor(model.n_layers)
        for v0, v1 in _tiles(model.vocab, LM_TILE):
            out.append(Instr(OP_LMHEAD, 0, v0, v1, 0, (LOGITS, (0, M, v0, v1)), [(XL, (0, M, 0, H))]))
        for b in range(M):
            out.append(Instr(OP_ARGMAX, 0, b, 0, 0, (NEXT, (b, b + 1, 0, 1)),
                             [(LOGITS, (b, b + 1, 0, model.vocab))]))
    return out


def _prefill_instrs(model, plan, S: int) -> List[Instr]:
    H, F, hd = model.hidden, model.ffn, model.head_dim
    nq, nkv, r = model.n_q_heads, model.n_kv_heads, model.group
    NQKV, NA = model.qkv_cols, model.attn_cols
    blocks = _tiles(S, plan.bm)
    out: List[Instr] = []
    for m, (m0, m1) in enumerate(blocks):
        out.append(Instr(OP_P_EMBED, 0, m, 0, 0, (0, (m0, m1, 0, H)), []))
    for l in range(model.n_layers):
        X = x_tensor(l)
        QKV, ATT = tensor_order(l, T_QKV), tensor_order(l, T_ATT)
        HR, ACT, XN = tensor_order(l, T_HRES), tensor_order(l, T_ACT), tensor_order(l, T_XNEXT)
        for m, (m0, m1) in enumerate(blocks):
            for n0, n1 in _tiles(NQKV, plan.bn):
                out.append(Instr(OP_P_QKV, l, m, n0, n1, (QKV, (m0, m1, n0, n1)), [(X, (m0, m1, 0, H))]))
        for m, (m0, m1) in enumerate(blocks):
            for h in range(nq):
                g = h // r
                out.append(Instr(OP_P_ATTN, l, m, h, 0, (ATT, (m0, m1, h * hd, (h + 1) * hd)),
                                 [(QKV, (m0, m1, h * hd, (h + 1) * hd)),
                                  (QKV, (0, m1, nq * hd + g * hd, nq * hd + (g + 1) * hd)),
                                  (QKV, (0, m1, (nq + nkv) * hd + g * hd, (nq + nkv) * hd + (g + 1) * hd))]))
        for m, (m0, m1) in enumerate(blocks):
            for n0, n1 in _tiles(H, plan.bn):
                out.append(Instr(OP_P_OPROJ, l, m, n0, n1, (HR, (m0, m1, n0, n1)),
                                 [(ATT, (m0, m1, 0, NA)), (X, (m0, m1, n0, n1))]))
        for m, (m0, m1) in enumerate(blocks):
            for n0, n1 in _tiles(F, plan.bn):
                out.append(Instr(OP_P_GATEUP, l, m, n0, n1, (ACT, (m0, m1, n0, n1)), [(HR, (m0, m1, 0, H))]))
        for m, (m0, m1) in enumerate(blocks):
            for n0, n1 in _tiles(H, plan.bn):
                out.append(Instr(OP_P_DOWN, l, m, n0, n1, (XN, (m0, m1, n0, n1)),
                                 [(ACT, (m0, m1, 0, F)), (HR, (m0, m1, n0, n1))]))
    return out


def build(model, plan, mode: int, rows: int, ctx_max: int) -> Queue:
    """Build the queue for ``rows`` decode rows (B) or prefill rows (S_max)."""
    _check(model, plan, mode, rows, ctx_max)
    NS = math.ceil(ctx_max / plan.kb) if mode == MODE_DECODE else 0
    instrs = (_decode_instrs(model, plan, rows, NS) if mode == MODE_DECODE
              else _prefill_instrs(model, plan, rows))
    fuse = getattr(plan, "fuse_combine", 0) if mode == MODE_DECODE else 0
    flags = (1 if fuse == 1 else 0) | (4 if fuse == 2 else 0)
    if getattr(plan, "loop", 0):
        flags |= 2
    if getattr(plan, "attn_pop", 0):
        flags |= 8                    # run-time hand-out of the splits: the same instructions
    q = Queue(mode, rows, ctx_max, NS, model.n_layers,
              (plan.tq, plan.to, plan.tf, plan.td, plan.kb, plan.bm, plan.bn), plan.n_queues, flags)

    # barriers: one per distinct written tile, numbered by first write
    tile_id: Dict[Tuple[int, Box], int] = {}
    for ins in instrs:
        if ins.write not in tile_id:
            tile_id[ins.write] = len(tile_id)
            q.tiles.append(ins.write)
            q.targets.append(0)
        ins.signal = tile_id[ins.write]
        q.targets[ins.signal] += 1
    if fuse == 2:
        # the merge of the last-arriving split signals each partial tile once more
        for ins in instrs:
            if ins.op == OP_ATTN and ins.a2 == 0:
                q.targets[ins.signal] += 1

    by_tensor: Dict[int, List[Tuple[Box, int]]] = {}
    for (t, box), bid in tile_id.items():
        by_tensor.setdefault(t, []).append((box, bid))

    # wait lists: every written tile intersecting a read region; the previous
    # step's tiles (loop queues) form ranges of their own, flagged, after them
    def wait_ranges(reads, flag):
        found = set()
        for t, rbox in reads:
            for box, bid in by_tensor.get(t, []):
                if _overlap(box, rbox):
                    found.add((t, box[2], box[0], bid))
        ws = [bid for (_, _, _, bid) in sorted(found)]
        ranges: List[Tuple[int, int]] = []
        for bid in ws:
            if ranges and ranges[-1][0] + ranges[-1][1] == bid:
                ranges[-1] = (ranges[-1][0], ranges[-1][1] + 1)
            else:
                ranges.append((bid, 1))
        return [(f, c | flag) for f, c in ranges], len(ws)

    for ins in instrs:
        same, n_same = wait_ranges(ins.reads, 0)
        prev, n_prev = wait_ranges(ins.prev_reads, PREV)
        ins.wait_off, ins.wait_cnt, ins.n_wait = len(q.waits), len(same) + len(prev), n_same + n_prev
        q.waits.extend(same + prev)
    q.instrs = instrs

    # maximal runs of one (op, layer), for launching one kernel per op
    for i, ins in enumerate(instrs):
        if q.segments and q.segments[-1][0] == ins.op and q.segments[-1][1] == ins.layer:
            op, layer, first, count = q.segments[-1]
            q.segments[-1] = (op, layer, first, count + 1)
        else:
            q.segments.append((ins.op, ins.layer, i, 1))
    return q
