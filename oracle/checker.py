"""Tile-dependency checker and CPU simulator of the interpreter (test infrastructure).

Two independent ways to show that a queue enforces every producer -> consumer
dependency on tiles of the intermediate tensors (MegaOps abstract; barriers as
tensors and the atomic-pop interpreter of the "Production Megakernels" lecture
summary):

``static_check``  decodes the serialised queue, rebuilds each instruction's
    write and read regions from its opcode and arguments as element masks (not
    boxes), and verifies that (1) every barrier's target equals the number of
    instructions that signal it (plus one for a split-partial tile whose last
    split merges, flags bit 2) and all of them write one tile, (2) every
    element an instruction reads that some instruction writes lies in a tile
    the instruction waits on, and it waits on nothing else, (3) every producer
    it waits on sits earlier in the queue, so a global pop in queue order can
    never deadlock, and (4) wait lists are in the documented order.

    For a loop queue (several decode steps in one launch) it also checks (5)
    that buffers can be reused across steps: every instruction must be an
    ancestor of some ARGMAX and a descendant of some EMBED tile of its step,
    through same-step waits, and every EMBED tile waits on all of the previous
    step's ARGMAX; then no instruction of step t + 1 can overwrite a tile
    before every reader of it in step t is done.

``simulate``  runs the queue with K virtual workers that pop in queue order
    (round-robin over sub-queues when the queue has several), block on their
    wait lists, and take random times; a loop queue runs T steps, the queue
    repeated T times, with counters that are never cleared (a same-step wait at
    step t needs target * (t + 1) signals, a previous-step wait target * t).
    Each instruction runs its tile body on float64 state that holds NaN until
    written, and every element carries the step that last wrote it; inputs are
    read when the body starts and outputs land when it ends.  Under flags bit 2
    the attention split whose signal completes its (row, KV head) merges the
    partials into the attention output as it ends and signals once more.  A read of an
    element not written in the expected step (unwritten, stale or already
    overwritten by the next step) is reported, as is a deadlock.  The result
    can be compared bit for bit across worker counts and schedules, and with
    the plain forward pass.
"""
from __future__ import annotations

import heapq
import math
import struct
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import numerics as N
from . import queue_spec as QS


# ----------------------------------------------------------------------------- decoding the bytes

@dataclass
class Parsed:
    mode: int
    n_instr: int
    n_barriers: int
    n_queues: int
    rows: int
    ctx_max: int
    n_splits: int
    n_layers: int
    plan: Tuple[int, ...]
    flags: int                   # bit 0: combines fused into the O-projection; 1: loop; 2: last split merges
    segments: List[Tuple[int, int, int, int]]
    instr: np.ndarray            # [n, 9] int64: op, layer, a0, a1, a2, wait_off, wait_cnt, signal, n_wait
    ranges: np.ndarray           # [n_ranges, 2]
    targets: np.ndarray          # [n_barriers]

    def waits_of(self, i: int, prev: bool = False) -> List[int]:
        """Barrier ids instruction i waits on in its own step (or, with
        ``prev``, the previous step's), in wait-list order."""
        off, cnt = int(self.instr[i, 5]), int(self.instr[i, 6])
        out: List[int] = []
        for f, c in self.ranges[off: off + cnt]:
            if bool(int(c) & QS.PREV) == prev:
                out.extend(range(int(f), int(f) + (int(c) & ~QS.PREV)))
        return out

    @property
    def loop(self) -> bool:
        return bool(self.flags & 2)

    @property
    def merge_last(self) -> bool:
        return bool(self.flags & 4)


def parse(parts: Dict[str, bytes]) -> Parsed:
    meta = parts["meta"]
    h = struct.unpack_from("<20I", meta, 0)
    if h[0] != QS.MAGIC or h[1] != QS.VERSION:
        raise ValueError("bad queue header")
    n_instr, n_bar, n_rng, n_seg = h[3], h[4], h[5], h[6]
    segs = [struct.unpack_from("<4I", meta, 80 + 16 * k) for k in range(n_seg)]
    if len(meta) != 80 + 16 * n_seg:
        raise ValueError("meta size")
    raw = parts["instr"]
    if len(raw) != 32 * n_instr:
        raise ValueError("instr size")
    rec = np.frombuffer(raw, dtype=np.dtype([("op", "<u2"), ("layer", "<u2"), ("f", "<u4", (7,))]))
    instr = np.empty((n_instr, 9), dtype=np.int64)
    instr[:, 0] = rec["op"]
    instr[:, 1] = rec["layer"]
    instr[:, 2:] = rec["f"]
    ranges = np.frombuffer(parts["waits"], dtype="<u4").reshape(-1, 2).astype(np.int64)
    targets = np.frombuffer(parts["targets"], dtype="<u4").astype(np.int64)
    if len(ranges) != n_rng or len(targets) != n_bar:
        raise ValueError("part sizes")
    return Parsed(h[2], n_instr, n_bar, h[7], h[8], h[9], h[10], h[11], tuple(h[12:19]), h[19], segs,
                  instr, ranges, targets)


# ----------------------------------------------------------------------------- regions as element masks

class Space:
    """Shapes of every intermediate tensor, indexed like the queue's tensor order."""

    def __init__(self, model, p: Parsed):
        self.model, self.p = model, p
        M, H, F = p.rows, model.hidden, model.ffn
        self.shapes: Dict[int, Tuple[int, int]] = {0: (M, H)}
        for l in range(model.n_layers):
            self.shapes[QS.tensor_order(l, QS.T_QKV)] = (M, model.qkv_cols)
            self.shapes[QS.tensor_order(l, QS.T_OPART)] = (M, model.n_kv_heads)
            self.shapes[QS.tensor_order(l, QS.T_ATT)] = (M, model.attn_cols)
            self.shapes[QS.tensor_order(l, QS.T_HRES)] = (M, H)
            self.shapes[QS.tensor_order(l, QS.T_ACT)] = (M, F)
            self.shapes[QS.tensor_order(l, QS.T_XNEXT)] = (M, H)
        if p.loop:
            self.shapes[QS.logits_tensor(model.n_layers)] = (M, model.vocab)
            self.shapes[QS.next_tensor(model.n_layers)] = (M, 1)

    def regions(self, op: int, layer: int, a0: int, a1: int, a2: int):
        """(write, reads, previous-step reads) as (tensor, row slice, col slice),
        rebuilt from the opcode."""
        w, reads = self._regions(op, layer, a0, a1, a2)
        prev = []
        if self.p.loop and op == QS.OP_EMBED:
            prev = [(QS.next_tensor(self.model.n_layers), slice(0, self.p.rows), slice(0, 1))]
        return w, reads, prev

    def _regions(self, op: int, layer: int, a0: int, a1: int, a2: int):
        m, p = self.model, self.p
        M, H, F, hd = p.rows, m.hidden, m.ffn, m.head_dim
        nq, nkv, r = m.n_q_heads, m.n_kv_heads, m.n_q_heads // m.n_kv_heads
        X, XN = QS.x_tensor(layer), QS.tensor_order(layer, QS.T_XNEXT)
        QKV, OP = QS.tensor_order(layer, QS.T_QKV), QS.tensor_order(layer, QS.T_OPART)
        ATT, HR = QS.tensor_order(layer, QS.T_ATT), QS.tensor_order(layer, QS.T_HRES)
        ACT = QS.tensor_order(layer, QS.T_ACT)
        allr = slice(0, M)
        kcol = lambda g: slice(nq * hd + g * hd, nq * hd + (g + 1) * hd)
        vcol = lambda g: slice((nq + nkv) * hd + g * hd, (nq + nkv) * hd + (g + 1) * hd)
        if op == QS.OP_EMBED:
            return (0, allr, slice(a0, a1)), []
        if op == QS.OP_QKV:
            return (QKV, allr, slice(a0, a1)), [(X, allr, slice(0, H))]
        if op == QS.OP_ATTN:
            b, g = a0, a1
            row = slice(b, b + 1)
            return (OP, row, slice(g, g + 1)), [(QKV, row, slice(g * r * hd, (g + 1) * r * hd)),
                                                (QKV, row, kcol(g)), (QKV, row, vcol(g))]
        if op == QS.OP_COMBINE:
            b, g = a0, a1
            return (ATT, slice(b, b + 1), slice(g * r * hd, (g + 1) * r * hd)), [(OP, slice(b, b + 1), slice(g, g + 1))]
        if op == QS.OP_OPROJ:
            # no combine instructions (flags bit 0 or 2): the wait is on the partial tiles
            att = (OP, allr, slice(0, nkv)) if p.flags & 5 else (ATT, allr, slice(0, nq * hd))
            return (HR, allr, slice(a0, a1)), [att, (X, allr, slice(a0, a1))]
        if op == QS.OP_GATEUP:
            return (ACT, allr, slice(a0, a1)), [(HR, allr, slice(0, H))]
        if op == QS.OP_DOWN:
            return (XN, allr, slice(a0, a1)), [(ACT, allr, slice(0, F)), (HR, allr, slice(a0, a1))]
        if op == QS.OP_LMHEAD and p.loop:
            XL, LG = QS.x_tensor(m.n_layers), QS.logits_tensor(m.n_layers)
            return (LG, allr, slice(a0, a1)), [(XL, allr, slice(0, H))]
        if op == QS.OP_ARGMAX and p.loop:
            LG, NX = QS.logits_tensor(m.n_layers), QS.next_tensor(m.n_layers)
            return (NX, slice(a0, a0 + 1), slice(0, 1)), [(LG, slice(a0, a0 + 1), slice(0, m.vocab))]
        bm = p.plan[5]
        rows = lambda mb: slice(mb * bm, min((mb + 1) * bm, M))
        upto = lambda mb: slice(0, min((mb + 1) * bm, M))
        if op == QS.OP_P_EMBED:
            return (0, rows(a0), slice(0, H)), []
        if op == QS.OP_P_QKV:
            return (QKV, rows(a0), slice(a1, a2)), [(X, rows(a0), slice(0, H))]
        if op == QS.OP_P_ATTN:
            h, g = a1, a1 // r
            return (ATT, rows(a0), slice(h * hd, (h + 1) * hd)), [
                (QKV, rows(a0), slice(h * hd, (h + 1) * hd)), (QKV, upto(a0), kcol(g)), (QKV, upto(a0), vcol(g))]
        if op == QS.OP_P_OPROJ:
            return (HR, rows(a0), slice(a1, a2)), [(ATT, rows(a0), slice(0, nq * hd)), (X, rows(a0), slice(a1, a2))]
        if op == QS.OP_P_GATEUP:
            return (ACT, rows(a0), slice(a1, a2)), [(HR, rows(a0), slice(0, H))]
        if op == QS.OP_P_DOWN:
            return (XN, rows(a0), slice(a1, a2)), [(ACT, rows(a0), slice(0, F)), (HR, rows(a0), slice(a1, a2))]
        raise ValueError(f"unknown opcode {op}")


def static_check(model, parts: Dict[str, bytes], max_errors: int = 20) -> List[str]:
    """Return a list of violations (empty when the queue is sound)."""
    p = parse(parts)
    sp = Space(model, p)
    errs: List[str] = []

    def err(msg):
        if len(errs) < max_errors:
            errs.append(msg)

    n = p.n_instr
    writer: Dict[int, np.ndarray] = {t: np.full(s, -1, dtype=np.int64) for t, s in sp.shapes.items()}
    signallers: Dict[int, List[int]] = {}
    regions = []
    for i in range(n):
        op, layer, a0, a1, a2, _, _, sig, _ = (int(v) for v in p.instr[i])
        if not 0 <= sig < p.n_barriers:
            err(f"instr {i}: signal {sig} out of range")
            regions.append(None)
            continue
        try:
            w, reads, prev_reads = sp.regions(op, layer, a0, a1, a2)
        except Exception as e:          # noqa: BLE001 -- report, do not crash the checker
            err(f"instr {i}: {e}")
            regions.append(None)
            continue
        regions.append((w, reads, prev_reads))
        signallers.setdefault(sig, []).append(i)
        t, rs, cs = w
        cur = writer[t][rs, cs]
        clash = (cur != -1) & (cur != sig)
        if np.any(clash):
            err(f"instr {i}: writes elements of another barrier's tile")
        writer[t][rs, cs] = sig

    # (1) targets and tile identity; with merges in the last split, a partial
    # tile is signalled once more by the merge
    opart = {QS.tensor_order(l, QS.T_OPART) for l in range(model.n_layers)}
    for bid in range(p.n_barriers):
        who = signallers.get(bid, [])
        extra = int(p.merge_last and bool(who) and regions[who[0]] is not None and regions[who[0]][0][0] in opart)
        if len(who) + extra != int(p.targets[bid]):
            err(f"barrier {bid}: target {int(p.targets[bid])} but {len(who)} signallers"
                + (" and a merge" if extra else ""))
        ws = {regions[i][0][0] for i in who if regions[i] is not None}
        if len(ws) > 1:
            err(f"barrier {bid}: signallers write different tensors")
    first_sig = {bid: min(who) for bid, who in signallers.items()}
    last_sig = {bid: max(who) for bid, who in signallers.items()}

    # tile boxes of each barrier, for the ordering rule
    bbox: Dict[int, Tuple[int, int, int]] = {}
    for t, wmap in writer.items():
        for bid in np.unique(wmap[wmap >= 0]):
            rr, cc = np.nonzero(wmap == bid)
            bbox[int(bid)] = (t, int(cc.min()), int(rr.min()))

    def needed(reads):
        need = set()
        for t, rs, cs in reads:
            ids = writer[t][rs, cs]
            need.update(int(v) for v in np.unique(ids[ids >= 0]))
        return need

    same_waits: List[List[int]] = [[] for _ in range(n)]
    for i in range(n):
        if regions[i] is None:
            continue
        _, reads, prev_reads = regions[i]
        try:
            waits, pwaits = p.waits_of(i), p.waits_of(i, prev=True)
        except Exception:                # noqa: BLE001
            err(f"instr {i}: wait ranges out of range")
            continue
        same_waits[i] = waits
        if int(p.instr[i, 8]) != len(waits) + len(pwaits):
            err(f"instr {i}: n_wait {int(p.instr[i, 8])} != {len(waits) + len(pwaits)}")
        if pwaits and not p.loop:
            err(f"instr {i}: previous-step waits in a single-step queue")
        for kind, lst, reg in (("", waits, reads), ("previous-step ", pwaits, prev_reads)):
            got, need = set(lst), needed(reg)
            if len(got) != len(lst):
                err(f"instr {i}: duplicate {kind}waits")
            missing, extra = need - got, got - need
            if missing:                                         # (2) coverage
                err(f"instr {i} ({QS.OP_NAMES.get(int(p.instr[i, 0]))}): missing {kind}waits {sorted(missing)[:5]}")
            if extra:
                err(f"instr {i}: {kind}waits on tiles it does not read {sorted(extra)[:5]}")
            for bid in got:
                if bid not in first_sig:
                    err(f"instr {i}: waits on barrier {bid} that nobody signals")
                elif not kind and last_sig[bid] >= i:           # (3) topological order
                    err(f"instr {i}: waits on barrier {bid} whose producer {last_sig[bid]} is not earlier")
            keys = [bbox.get(b, (0, 0, 0)) for b in lst]        # (4) documented order
            if keys != sorted(keys):
                err(f"instr {i}: {kind}wait list out of order")

    if p.loop:                                                  # (5) reuse across steps
        ops = p.instr[:, 0]
        from_embed = [False] * n
        consumers: List[List[int]] = [[] for _ in range(n)]
        for i in range(n):
            prods = [j for b in same_waits[i] for j in signallers.get(b, []) if j < i]
            for j in prods:
                consumers[j].append(i)
            from_embed[i] = int(ops[i]) == QS.OP_EMBED or any(from_embed[j] for j in prods)
        to_argmax = [False] * n
        for i in reversed(range(n)):
            to_argmax[i] = int(ops[i]) == QS.OP_ARGMAX or any(to_argmax[c] for c in consumers[i])
        for i in range(n):
            if not from_embed[i]:
                err(f"instr {i}: descends from no embedding tile of its step (may overwrite a tile the "
                    f"previous step still reads)")
            if not to_argmax[i]:
                err(f"instr {i}: leads to no argmax of its step (the next step may overwrite what it reads)")
    return errs


# ----------------------------------------------------------------------------- tile bodies and simulation

class DecodeState:
    """Float64 intermediate tensors of a run of decode steps, NaN until written.
    Every element records the step that last wrote it (-1: never)."""

    def __init__(self, model: N.Model, p: Parsed, K: np.ndarray, V: np.ndarray,
                 ctx_lens: Sequence[int], tokens=None, x0=None, feedback: bool = False):
        cfg = model.cfg
        self.model, self.cfg, self.p = model, cfg, p
        self.K, self.V, self.ctx = K, V, [int(c) for c in ctx_lens]
        sp = Space(cfg, p)
        self.t = {t: np.full(s, np.nan) for t, s in sp.shapes.items()}
        self.ver = {t: np.full(s, -1, dtype=np.int64) for t, s in sp.shapes.items()}
        # split partials: [M, nkv, NS, r, hd + 2]  (o | m | l), and the step of each slot
        r = cfg.n_q_heads // cfg.n_kv_heads
        self.opart = {l: np.full((p.rows, cfg.n_kv_heads, p.n_splits, r, cfg.head_dim + 2), np.nan)
                      for l in range(cfg.n_layers)}
        self.opart_ver = {l: np.full((p.rows, cfg.n_kv_heads, p.n_splits), -1, dtype=np.int64)
                          for l in range(cfg.n_layers)}
        if not cfg.has_embed:
            self.t[0][:] = x0
            self.ver[0][:] = 0
        # token ids: [B] for one step, or [steps][B] (teacher-forced, or the first row only
        # when the argmax feeds the next step)
        self.tokens = None if tokens is None else np.atleast_2d(np.asarray(tokens))
        self.feedback = feedback
        self.logits: Dict[int, np.ndarray] = {}       # step -> [M, V] (loop queues)
        self.next: Dict[int, np.ndarray] = {}         # step -> [M]
        self.bad_reads: List[str] = []

    def read(self, i: int, step: int, t: int, rs: slice, cs: slice, want: int) -> np.ndarray:
        if not np.all(self.ver[t][rs, cs] == want):
            self.bad_reads.append(f"instr {i} (step {step}) read elements of tensor {t} not written in step {want}")
        return self.t[t][rs, cs].copy()

    def body(self, i: int, step: int = 0, merge: bool = False):
        """Compute instruction i of `step` from the current state; returns a commit
        closure.  ``merge``: the split merge that attention instruction i performs
        when it arrives last at its (row, KV head)."""
        op, l, a0, a1, a2 = (int(v) for v in self.p.instr[i, :5])
        if merge:
            op = -op
        cfg, lw = self.cfg, (self.model.layers[l] if self.model.layers else None)
        M, H, hd = self.p.rows, cfg.hidden, cfg.head_dim
        nq, nkv = cfg.n_q_heads, cfg.n_kv_heads
        r = nq // nkv
        X = QS.x_tensor(l)
        QKV, OPT = QS.tensor_order(l, QS.T_QKV), QS.tensor_order(l, QS.T_OPART)
        ATT, HR = QS.tensor_order(l, QS.T_ATT), QS.tensor_order(l, QS.T_HRES)
        ACT, XN = QS.tensor_order(l, QS.T_ACT), QS.tensor_order(l, QS.T_XNEXT)
        rd = lambda t, rs, cs: self.read(i, step, t, rs, cs, step)

        def put(t, rs, cs, val, also=None):
            def commit():
                self.t[t][rs, cs] = val
                self.ver[t][rs, cs] = step
                if also:
                    also()
            return commit

        def merged(b, g):
            """The merged attention output of (row b, KV head g), NaN if a split
            partial was not written in this step."""
            if not np.all(self.opart_ver[l][b, g] == step):
                self.bad_reads.append(f"instr {i} (step {step}) read split partials not written in step {step}")
                return np.full(r * hd, np.nan)
            slots = self.opart[l][b, g]                     # [NS, r, hd + 2] = (o | m | l)
            if np.any(np.isnan(slots)):                     # computed from unwritten inputs upstream
                return np.full(r * hd, np.nan)
            return N.combine_splits([(sl[:, :hd], sl[:, hd], sl[:, hd + 1]) for sl in slots]).reshape(-1)

        if op == QS.OP_EMBED:
            if self.feedback and step > 0:
                NX = QS.next_tensor(cfg.n_layers)
                got = self.read(i, step, NX, slice(0, M), slice(0, 1), step - 1)[:, 0]
                if not np.all(np.isfinite(got)):               # not written yet: reported above
                    return put(0, slice(0, M), slice(a0, a1), np.full((M, a1 - a0), np.nan))
                tok = got.astype(np.int64)
            else:
                tok = self.tokens[step]
            return put(0, slice(0, M), slice(a0, a1), self.model.embed[np.asarray(tok)][:, a0:a1])
        if op == QS.OP_QKV:
            xn = N.rms_norm(rd(X, slice(0, M), slice(0, H)), lw.attn_norm, cfg.rms_eps)
            return put(QKV, slice(0, M), slice(a0, a1), xn @ lw.wqkv[a0:a1].T)
        if op == QS.OP_ATTN:
            b, g, s = a0, a1, a2
            row = slice(b, b + 1)
            q = rd(QKV, row, slice(g * r * hd, (g + 1) * r * hd)).reshape(r, hd)
            k = rd(QKV, row, slice(nq * hd + g * hd, nq * hd + (g + 1) * hd)).reshape(hd)
            v = rd(QKV, row, slice((nq + nkv) * hd + g * hd, (nq + nkv) * hd + (g + 1) * hd)).reshape(hd)
            if cfg.qk_norm:
                q = N.rms_norm(q, lw.q_norm, cfg.rms_eps)
                k = N.rms_norm(k, lw.k_norm, cfg.rms_eps)
            pos = self.ctx[b] + step
            q, k = N.rope(q, pos, cfg.rope_theta), N.rope(k, pos, cfg.rope_theta)
            kb = self.p.plan[4]
            j0, j1 = s * kb, min((s + 1) * kb, pos + 1)
            if j0 <= pos < j1:                      # this split holds the new token
                self.K[l, b, g, pos] = N.store_like(k, self.K.dtype)
                self.V[l, b, g, pos] = N.store_like(v, self.V.dtype)
            Ks = N.to_f64(self.K[l, b, g, j0:max(j0, j1)])
            Vs = N.to_f64(self.V[l, b, g, j0:max(j0, j1)])
            o, m, lsum = N.attention_split(q, Ks, Vs)
            part = np.concatenate([o, m[:, None], lsum[:, None]], axis=1)     # (o | m | l)

            def commit():
                self.opart[l][b, g, s] = part
                self.opart_ver[l][b, g, s] = step
                if np.all(self.opart_ver[l][b, g] == step):
                    self.t[OPT][b, g] = 0.0
                    self.ver[OPT][b, g] = step
            return commit
        if op == QS.OP_COMBINE:
            b, g = a0, a1
            return put(ATT, slice(b, b + 1), slice(g * r * hd, (g + 1) * r * hd), merged(b, g)[None, :])
        if op == -QS.OP_ATTN:
            # the merge of (row b, KV head g) by its last-arriving split (flags bit 2)
            b, g = a0, a1
            return put(ATT, slice(b, b + 1), slice(g * r * hd, (g + 1) * r * hd), merged(b, g)[None, :])
        if op == QS.OP_OPROJ:
            if self.p.flags & 1:
                # fused: merge every (row, KV head)'s split partials here
                att = np.empty((M, nq * hd))
                for b in range(M):
                    for g in range(nkv):
                        att[b, g * r * hd:(g + 1) * r * hd] = merged(b, g)
            else:
                att = rd(ATT, slice(0, M), slice(0, nq * hd))
            xres = rd(X, slice(0, M), slice(a0, a1))
            return put(HR, slice(0, M), slice(a0, a1), xres + att @ lw.wo[a0:a1].T)
        if op == QS.OP_GATEUP:
            hn = N.rms_norm(rd(HR, slice(0, M), slice(0, H)), lw.ffn_norm, cfg.rms_eps)
            val = N.silu(hn @ lw.wgate[a0:a1].T) * (hn @ lw.wup[a0:a1].T)
            return put(ACT, slice(0, M), slice(a0, a1), val)
        if op == QS.OP_DOWN:
            a = rd(ACT, slice(0, M), slice(0, cfg.ffn))
            hres = rd(HR, slice(0, M), slice(a0, a1))
            return put(XN, slice(0, M), slice(a0, a1), hres + a @ lw.wdown[a0:a1].T)
        if op == QS.OP_LMHEAD:
            XL, LG = QS.x_tensor(cfg.n_layers), QS.logits_tensor(cfg.n_layers)
            val = N.lm_head(cfg, rd(XL, slice(0, M), slice(0, H)), self.model.final_norm, self.model.lm_head[a0:a1])

            def keep():
                self.logits.setdefault(step, np.full((M, cfg.vocab), np.nan))[:, a0:a1] = val
            return put(LG, slice(0, M), slice(a0, a1), val, keep)
        if op == QS.OP_ARGMAX:
            b = a0
            LG, NX = QS.logits_tensor(cfg.n_layers), QS.next_tensor(cfg.n_layers)
            idx = int(N.argmax_lowest(rd(LG, slice(b, b + 1), slice(0, cfg.vocab)))[0])

            def keep():
                self.next.setdefault(step, np.full(M, -1, dtype=np.int64))[b] = idx
            return put(NX, slice(b, b + 1), slice(0, 1), np.array([[float(idx)]]), keep)
        raise ValueError(f"opcode {op} has no decode tile body")


@dataclass
class SimResult:
    deadlock: bool
    bad_reads: List[str]
    x_out: np.ndarray
    counters: np.ndarray
    state: DecodeState
    order: List[Tuple[int, int]]        # (step, instruction) in start order


def simulate(model: N.Model, parts: Dict[str, bytes], K: np.ndarray, V: np.ndarray,
             ctx_lens: Sequence[int], workers: int, seed: int, tokens=None, x0=None,
             reverse_ties: bool = False, steps: int = 1, feedback: bool = False) -> SimResult:
    """Event simulation of ``workers`` interpreters executing ``steps`` decode
    steps of the queue (more than one only for a loop queue): the queue's
    instructions repeated ``steps`` times, sub-queue k holding positions
    k, k + n_queues, ... of that sequence.  Step t of row b sits at position
    ctx_lens[b] + t; with ``feedback`` each step after the first embeds the
    previous step's argmax, otherwise ``tokens[t]``."""
    p = parse(parts)
    if steps > 1 and not p.loop:
        raise ValueError("only a loop queue runs several steps in one launch")
    st = DecodeState(model, p, K, V, ctx_lens, tokens, x0, feedback)
    rng = np.random.Generator(np.random.PCG64(seed))
    nq_ = max(1, p.n_queues)
    heads = [0] * nq_
    counters = np.zeros(p.n_barriers, dtype=np.int64)
    waits = [p.waits_of(i) for i in range(p.n_instr)]
    pwaits = [p.waits_of(i, prev=True) for i in range(p.n_instr)]
    total = steps * p.n_instr

    def pop(w):
        qi = w % nq_
        # sub-queue qi holds positions qi, qi + nq_, qi + 2 nq_, ... of the repeated queue
        k = qi + heads[qi] * nq_
        heads[qi] += 1
        return (k // p.n_instr, k % p.n_instr) if k < total else None

    def ready(step, i):
        return (all(counters[b] >= p.targets[b] * (step + 1) for b in waits[i]) and
                all(counters[b] >= p.targets[b] * step for b in pwaits[i]))

    now = 0.0
    events: List[Tuple[float, int, int, Tuple[int, int]]] = []   # (end time, tiebreak, worker, (step, instr))
    pending: Dict[Tuple[int, Tuple[int, int]], object] = {}
    waiting: Dict[int, Tuple[int, int]] = {}
    started: List[Tuple[int, int]] = []
    seq = 0
    for w in range(workers):
        job = pop(w)
        if job is not None:
            waiting[w] = job
    while True:
        # start every waiting worker whose barriers are complete (inputs read now)
        progressed = True
        while progressed:
            progressed = False
            for w in sorted(waiting, reverse=reverse_ties):
                step, i = waiting[w]
                if ready(step, i):
                    pending[(w, (step, i))] = st.body(i, step)
                    del waiting[w]
                    started.append((step, i))
                    seq += 1
                    heapq.heappush(events, (now + float(rng.uniform(0.2, 2.0)), seq, w, (step, i)))
                    progressed = True
        if not events:
            break
        # the earliest running instruction ends: outputs land, then its barrier is signalled
        now, _, w, job = heapq.heappop(events)
        pending.pop((w, job))()
        sig = int(p.instr[job[1], 7])
        counters[sig] += 1
        if (p.merge_last and int(p.instr[job[1], 0]) == QS.OP_ATTN
                and counters[sig] == p.targets[sig] * (job[0] + 1) - 1):
            # the last split of its (row, KV head): merge, then signal the tile again
            st.body(job[1], job[0], merge=True)()
            counters[sig] += 1
        nxt = pop(w)
        if nxt is not None:
            waiting[w] = nxt
    deadlock = bool(waiting) or len(started) != total
    x_out = st.t[QS.x_tensor(model.cfg.n_layers)]
    return SimResult(deadlock, st.bad_reads, x_out, counters, st, started)
