// Host builder of the instruction queue and its tile barriers.
//
// The queue is the work list of the on-device interpreter ("Production
// Megakernels" lecture summary, Technical details: a global instruction queue
// in DRAM that cores pop atomically).  It is built once per (model, plan) with
// the context length kept symbolic (Key takeaways: symbolic shapes, a single
// work queue): decode attention is split into NS = ceil(ctx_max / kb) key
// splits whatever the runtime context, and prefill row blocks past the runtime
// prompt length become no-ops.  Each instruction writes one tile of one
// intermediate tensor and waits on the barrier counters of exactly the tiles
// it reads (MegaOps abstract: dependencies on tiles of the intermediate
// tensor; Key takeaways: barriers as tensors partitioned by dependency).
//
// Barrier ids and wait lists are computed here by tile-index arithmetic: every
// tensor's tiles get a contiguous block of ids in the order the queue first
// writes them, and a reader's wait list is the union of the tile-index
// intervals its read region overlaps, sorted by (tensor, column, row) and
// stored as runs of consecutive ids.
#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "queue.h"

namespace mk {

namespace {

thread_local char g_err[512];

inline uint32_t cdiv(uint32_t a, uint32_t b) { return (a + b - 1) / b; }

// Append ids to a wait list, merging runs of consecutive ids into one range.
struct WaitBuilder {
  std::vector<Range>* out;
  uint32_t first_range;
  uint32_t n = 0;
  void add(uint32_t id) {
    ++n;
    if (out->size() > first_range) {
      Range& r = out->back();
      if (r.first + r.count == id) { ++r.count; return; }
    }
    out->push_back(Range{id, 1});
  }
  void add_run(uint32_t id, uint32_t count) { for (uint32_t k = 0; k < count; ++k) add(id + k); }
};

struct Builder {
  mk_queue* q;
  const mk_config& c;
  const mk_plan& p;

  // `prev_runs` (loop queues): barriers of the previous step, stored as their
  // own ranges after the same-step ones, with kPrevStep set in the count.
  void emit(uint16_t op, uint32_t layer, uint32_t a0, uint32_t a1, uint32_t a2, uint32_t signal,
            const std::vector<std::pair<uint32_t, uint32_t>>& runs,
            const std::vector<std::pair<uint32_t, uint32_t>>& prev_runs = {}) {
    Instr in{};
    in.op = op;
    in.layer = static_cast<uint16_t>(layer);
    in.a0 = a0; in.a1 = a1; in.a2 = a2;
    in.signal = signal;
    WaitBuilder wb{&q->waits, static_cast<uint32_t>(q->waits.size())};
    for (auto& r : runs) wb.add_run(r.first, r.second);
    WaitBuilder wp{&q->waits, static_cast<uint32_t>(q->waits.size())};
    for (auto& r : prev_runs) wp.add_run(r.first, r.second);
    for (size_t k = wp.first_range; k < q->waits.size(); ++k) q->waits[k].count |= kPrevStep;
    in.wait_off = wb.first_range;
    in.wait_cnt = static_cast<uint32_t>(q->waits.size()) - wb.first_range;
    in.n_wait = wb.n + wp.n;
    q->instr.push_back(in);
  }

  void decode() {
    const uint32_t M = p.rows, H = c.hidden, F = c.ffn, hd = c.head_dim;
    const uint32_t nq = c.n_q_heads, nkv = c.n_kv_heads, r = nq / nkv;
    const uint32_t NQKV = (nq + 2 * nkv) * hd;
    const uint32_t NS = cdiv(p.ctx_max, p.kb);
    q->n_splits = NS;
    const uint32_t nX = cdiv(H, p.td), nQ = cdiv(NQKV, p.tq), nO = cdiv(H, p.to), nF = cdiv(F, p.tf);
    const uint32_t L0 = c.has_embed ? nX : 0;
    // fused: the split combines are dropped and each O-projection tile waits on
    // the split partials' tiles (no attention-output tiles).  fuse_combine 1:
    // the O-projection merges the partials itself.  2: the split whose signal
    // completes a (row, KV head) merges them into the attention output and
    // signals that tile once more, so its target is NS + 1.
    const bool fused = p.fuse_combine != 0;
    const uint32_t natt = fused ? 0 : M * nkv;
    const uint32_t per_layer = nQ + M * nkv + natt + nO + nF + nX;
    auto qkv_id = [&](uint32_t l, uint32_t n) { return L0 + l * per_layer + n; };
    auto op_id = [&](uint32_t l, uint32_t b, uint32_t g) { return qkv_id(l, nQ) + b * nkv + g; };
    auto att_id = [&](uint32_t l, uint32_t g, uint32_t b) { return qkv_id(l, nQ) + M * nkv + g * M + b; };
    auto hres_id = [&](uint32_t l, uint32_t n) { return qkv_id(l, nQ) + M * nkv + natt + n; };
    auto act_id = [&](uint32_t l, uint32_t n) { return hres_id(l, nO) + n; };
    auto xn_id = [&](uint32_t l, uint32_t n) { return act_id(l, nF) + n; };
    auto x_exists = [&](uint32_t l) { return l > 0 || c.has_embed; };
    auto x_id = [&](uint32_t l, uint32_t n) { return l == 0 ? n : xn_id(l - 1, n); };

    // loop queues: LM-head tiles and one argmax per row after the layers
    const bool loop = p.loop != 0;
    const uint32_t nV = loop ? cdiv(c.vocab, kLmTile) : 0, nN = loop ? M : 0;
    const uint32_t tail = L0 + c.n_layers * per_layer;
    auto logits_id = [&](uint32_t j) { return tail + j; };
    auto next_id = [&](uint32_t b) { return tail + nV + b; };
    const uint32_t n_bar = tail + nV + nN;
    q->targets.assign(n_bar, 1);

    if (c.has_embed)
      for (uint32_t n = 0; n < nX; ++n) {
        std::vector<std::pair<uint32_t, uint32_t>> prev;
        if (loop) prev.push_back({next_id(0), M});
        emit(OP_EMBED, 0, n * p.td, std::min((n + 1) * p.td, H), 0, n, {}, prev);
      }
    for (uint32_t l = 0; l < (uint32_t)c.n_layers; ++l) {
      for (uint32_t n = 0; n < nQ; ++n) {
        std::vector<std::pair<uint32_t, uint32_t>> w;
        if (x_exists(l)) w.push_back({x_id(l, 0), nX});
        emit(OP_QKV, l, n * p.tq, std::min((n + 1) * p.tq, NQKV), 0, qkv_id(l, n), w);
      }
      // Splits are emitted split-major, the (row, KV head) pairs rotated by one
      // row per split, so that a worker's share of a layer's splits spans
      // several rows: with ragged contexts the later splits of a row are short
      // or empty, and a worker holding one split index for many rows would
      // hold only full or only empty splits.
      const uint32_t P = M * nkv;
      std::vector<std::vector<std::pair<uint32_t, uint32_t>>> att_waits(P);
      for (uint32_t b = 0; b < M; ++b)
        for (uint32_t g = 0; g < nkv; ++g) {
          // column intervals of q (group g), k_g and v_g, as QKV tile-index intervals
          uint32_t c0[3] = {g * r * hd, nq * hd + g * hd, (nq + nkv) * hd + g * hd};
          uint32_t c1[3] = {(g + 1) * r * hd, nq * hd + (g + 1) * hd, (nq + nkv) * hd + (g + 1) * hd};
          std::vector<std::pair<uint32_t, uint32_t>> tiles;   // [t0, t1] inclusive, merged
          for (int k = 0; k < 3; ++k) {
            uint32_t t0 = c0[k] / p.tq, t1 = (c1[k] - 1) / p.tq;
            if (!tiles.empty() && t0 <= tiles.back().second + 1)
              tiles.back().second = std::max(tiles.back().second, t1);
            else
              tiles.push_back({t0, t1});
          }
          for (auto& t : tiles) att_waits[b * nkv + g].push_back({qkv_id(l, t.first), t.second - t.first + 1});
          q->targets[op_id(l, b, g)] = p.fuse_combine == 2 ? NS + 1 : NS;
        }
      for (uint32_t s = 0; s < NS; ++s)
        for (uint32_t t = 0; t < P; ++t) {
          const uint32_t pr = (t + s * nkv) % P, b = pr / nkv, g = pr % nkv;
          emit(OP_ATTN, l, b, g, s, op_id(l, b, g), att_waits[pr]);
        }
      if (!fused)
        for (uint32_t g = 0; g < nkv; ++g)
          for (uint32_t b = 0; b < M; ++b)
            emit(OP_COMBINE, l, b, g, 0, att_id(l, g, b), {{op_id(l, b, g), 1}});
      for (uint32_t n = 0; n < nO; ++n) {
        uint32_t n0 = n * p.to, n1 = std::min((n + 1) * p.to, H);
        std::vector<std::pair<uint32_t, uint32_t>> w;
        if (x_exists(l)) w.push_back({x_id(l, n0 / p.td), (n1 - 1) / p.td - n0 / p.td + 1});
        if (fused) {
          // split-partial tiles in (KV head, row) order, as the reads sort
          for (uint32_t g = 0; g < nkv; ++g)
            for (uint32_t b = 0; b < M; ++b) w.push_back({op_id(l, b, g), 1});
        } else {
          w.push_back({att_id(l, 0, 0), nkv * M});
        }
        emit(OP_OPROJ, l, n0, n1, 0, hres_id(l, n), w);
      }
      for (uint32_t n = 0; n < nF; ++n)
        emit(OP_GATEUP, l, n * p.tf, std::min((n + 1) * p.tf, F), 0, act_id(l, n), {{hres_id(l, 0), nO}});
      for (uint32_t n = 0; n < nX; ++n) {
        uint32_t n0 = n * p.td, n1 = std::min((n + 1) * p.td, H);
        emit(OP_DOWN, l, n0, n1, 0, xn_id(l, n),
             {{hres_id(l, n0 / p.to), (n1 - 1) / p.to - n0 / p.to + 1}, {act_id(l, 0), nF}});
      }
    }
    if (loop) {
      for (uint32_t j = 0; j < nV; ++j)
        emit(OP_LMHEAD, 0, j * kLmTile, std::min((j + 1) * kLmTile, (uint32_t)c.vocab), 0, logits_id(j),
             {{x_id(c.n_layers, 0), nX}});
      for (uint32_t b = 0; b < M; ++b) emit(OP_ARGMAX, 0, b, 0, 0, next_id(b), {{logits_id(0), nV}});
    }
  }

  void prefill() {
    const uint32_t S = p.rows, H = c.hidden, F = c.ffn, hd = c.head_dim;
    const uint32_t nq = c.n_q_heads, nkv = c.n_kv_heads, r = nq / nkv;
    const uint32_t NQKV = (nq + 2 * nkv) * hd;
    const uint32_t nM = cdiv(S, p.bm), nQ = cdiv(NQKV, p.bn), nO = cdiv(H, p.bn), nF = cdiv(F, p.bn);
    const uint32_t nD = nO;
    q->n_splits = 0;
    const uint32_t per_layer = nM * (nQ + nq + nO + nF + nD);
    auto qkv_id = [&](uint32_t l, uint32_t m, uint32_t n) { return nM + l * per_layer + m * nQ + n; };
    auto att_id = [&](uint32_t l, uint32_t m, uint32_t h) { return qkv_id(l, nM, 0) + m * nq + h; };
    auto hres_id = [&](uint32_t l, uint32_t m, uint32_t n) { return att_id(l, nM, 0) + m * nO + n; };
    auto act_id = [&](uint32_t l, uint32_t m, uint32_t n) { return hres_id(l, nM, 0) + m * nF + n; };
    auto xn_id = [&](uint32_t l, uint32_t m, uint32_t n) { return act_id(l, nM, 0) + m * nD + n; };
    q->targets.assign(nM + c.n_layers * per_layer, 1);

    for (uint32_t m = 0; m < nM; ++m) emit(OP_P_EMBED, 0, m, 0, 0, m, {});
    for (uint32_t l = 0; l < (uint32_t)c.n_layers; ++l) {
      // rows of block m of X_l: one embedding tile, or every column tile of the previous layer
      auto x_row = [&](uint32_t m) -> std::pair<uint32_t, uint32_t> {
        return l == 0 ? std::make_pair(m, 1u) : std::make_pair(xn_id(l - 1, m, 0), nD);
      };
      auto x_cols = [&](uint32_t m, uint32_t n) -> std::pair<uint32_t, uint32_t> {
        return l == 0 ? std::make_pair(m, 1u) : std::make_pair(xn_id(l - 1, m, n), 1u);
      };
      for (uint32_t m = 0; m < nM; ++m)
        for (uint32_t n = 0; n < nQ; ++n)
          emit(OP_P_QKV, l, m, n * p.bn, std::min((n + 1) * p.bn, NQKV), qkv_id(l, m, n), {x_row(m)});
      for (uint32_t m = 0; m < nM; ++m)
        for (uint32_t h = 0; h < nq; ++h) {
          uint32_t g = h / r;
          uint32_t tq_ = (h * hd) / p.bn, tk = (nq * hd + g * hd) / p.bn, tv = ((nq + nkv) * hd + g * hd) / p.bn;
          // (column tile, row block) of q (block m) and of k, v (blocks 0..m); a tile can hold
          // both query and key columns, so de-duplicate, then order by column, then row
          std::vector<std::pair<uint32_t, uint32_t>> tiles;
          tiles.push_back({tq_, m});
          for (uint32_t mm = 0; mm <= m; ++mm) { tiles.push_back({tk, mm}); tiles.push_back({tv, mm}); }
          std::sort(tiles.begin(), tiles.end());
          tiles.erase(std::unique(tiles.begin(), tiles.end()), tiles.end());
          std::vector<std::pair<uint32_t, uint32_t>> w;
          for (auto& t : tiles) w.push_back({qkv_id(l, t.second, t.first), 1});
          emit(OP_P_ATTN, l, m, h, 0, att_id(l, m, h), w);
        }
      for (uint32_t m = 0; m < nM; ++m)
        for (uint32_t n = 0; n < nO; ++n)
          emit(OP_P_OPROJ, l, m, n * p.bn, std::min((n + 1) * p.bn, H), hres_id(l, m, n),
               {x_cols(m, n), {att_id(l, m, 0), nq}});
      for (uint32_t m = 0; m < nM; ++m)
        for (uint32_t n = 0; n < nF; ++n)
          emit(OP_P_GATEUP, l, m, n * p.bn, std::min((n + 1) * p.bn, F), act_id(l, m, n),
               {{hres_id(l, m, 0), nO}});
      for (uint32_t m = 0; m < nM; ++m)
        for (uint32_t n = 0; n < nD; ++n)
          emit(OP_P_DOWN, l, m, n * p.bn, std::min((n + 1) * p.bn, H), xn_id(l, m, n),
               {{hres_id(l, m, n), 1}, {act_id(l, m, 0), nF}});
    }
  }

  void segments() {
    for (uint32_t i = 0; i < q->instr.size(); ++i) {
      const Instr& in = q->instr[i];
      if (!q->segments.empty() && q->segments.back().op == in.op && q->segments.back().layer == in.layer)
        ++q->segments.back().count;
      else
        q->segments.push_back(Segment{in.op, in.layer, i, 1});
    }
  }
};

const char* validate(const mk_config& c, const mk_plan& p) {
  if (c.n_layers <= 0 || c.hidden <= 0 || c.n_q_heads <= 0 || c.n_kv_heads <= 0 || c.head_dim <= 0 || c.ffn <= 0)
    return "model dimensions must be positive";
  if (c.n_q_heads % c.n_kv_heads) return "query heads must be a multiple of KV heads";
  if (c.head_dim % 2) return "head_dim must be even (rotary pairs)";
  if (c.has_embed && c.vocab <= 0) return "an embedding needs a vocabulary";
  if (c.has_lm_head && c.vocab <= 0) return "an LM head needs a vocabulary";
  if (c.n_layers > 65535) return "too many layers";
  if (p.rows <= 0 || p.ctx_max <= 0) return "rows and ctx_max must be positive";
  if (p.n_queues < 1 || p.n_queues > kMaxQueues) return "n_queues out of range";
  if (p.fuse_combine < 0 || p.fuse_combine > 2) return "fuse_combine must be 0, 1 or 2";
  if (p.loop != 0 && p.loop != 1) return "loop must be 0 or 1";
  if (p.attn_pop != 0 && p.attn_pop != 1) return "attn_pop must be 0 or 1";
  if (p.attn_pop && (p.mode != MK_DECODE || p.loop)) return "attn_pop is for single-step decode queues";
  if (p.loop && (p.mode != MK_DECODE || !c.has_embed || !c.has_lm_head))
    return "a loop queue decodes a model with an embedding and an LM head";
  if (p.mode == MK_DECODE) {
    if (p.rows > kMaxDecodeRows) return "decode rows above the maximum";
    if (std::min({p.tq, p.to, p.tf, p.td, p.kb}) <= 0) return "tile sizes must be positive";
  } else if (p.mode == MK_PREFILL) {
    if (std::min(p.bm, p.bn) <= 0) return "tile sizes must be positive";
    if (p.bn % c.head_dim) return "prefill column tile must hold whole heads";
    if (p.rows > p.ctx_max) return "prefill rows exceed the cache";
  } else {
    return "unknown mode";
  }
  return nullptr;
}

}  // namespace

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

const char* last_error() { return g_err; }

}  // namespace mk

extern "C" {

mk_status mk_build_queue(const mk_config* cfg, const mk_plan* plan, mk_queue** out) {
  if (!cfg || !plan || !out) { mk::set_error("null argument"); return MK_EINVAL; }
  *out = nullptr;
  if (const char* why = mk::validate(*cfg, *plan)) { mk::set_error("%s", why); return MK_EINVAL; }
  mk_queue* q = new (std::nothrow) mk_queue();
  if (!q) { mk::set_error("out of host memory"); return MK_ENOMEM; }
  try {
    static std::atomic<uint64_t> next_serial{1};
    q->serial = next_serial.fetch_add(1);
    q->cfg = *cfg;
    q->plan = *plan;
    mk::Builder b{q, q->cfg, q->plan};
    if (plan->mode == MK_DECODE) b.decode(); else b.prefill();
    b.segments();
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    q->dev_instr_off = 0;
    q->dev_waits_off = up(q->instr.size() * sizeof(mk::Instr));
    q->dev_targets_off = q->dev_waits_off + up(q->waits.size() * sizeof(mk::Range));
    q->dev_bytes = q->dev_targets_off + up(q->targets.size() * sizeof(uint32_t));
  } catch (const std::bad_alloc&) {
    delete q;
    mk::set_error("out of host memory");
    return MK_ENOMEM;
  }
  *out = q;
  return MK_OK;
}

size_t mk_queue_nbytes(const mk_queue* q, int32_t part) {
  if (!q) return 0;
  switch (part) {
    case MK_PART_META: return 80 + 16 * q->segments.size();
    case MK_PART_INSTR: return q->instr.size() * sizeof(mk::Instr);
    case MK_PART_WAITS: return q->waits.size() * sizeof(mk::Range);
    case MK_PART_TARGETS: return q->targets.size() * sizeof(uint32_t);
    case MK_PART_DEVICE: return q->dev_bytes;
    default: return 0;
  }
}

mk_status mk_queue_export(const mk_queue* q, int32_t part, void* host_dst, size_t nbytes) {
  if (!q || !host_dst) { mk::set_error("null argument"); return MK_EINVAL; }
  size_t need = mk_queue_nbytes(q, part);
  if (part < MK_PART_META || part > MK_PART_DEVICE) { mk::set_error("unknown part %d", part); return MK_EINVAL; }
  if (nbytes != need) { mk::set_error("part %d needs %zu bytes, got %zu", part, need, nbytes); return MK_EINVAL; }
  auto* d = static_cast<uint8_t*>(host_dst);
  const mk_plan& p = q->plan;
  switch (part) {
    case MK_PART_META: {
      uint32_t h[20] = {mk::kMagic, mk::kVersion, (uint32_t)p.mode, (uint32_t)q->instr.size(),
                        (uint32_t)q->targets.size(), (uint32_t)q->waits.size(),
                        (uint32_t)q->segments.size(), (uint32_t)p.n_queues, (uint32_t)p.rows,
                        (uint32_t)p.ctx_max, q->n_splits, (uint32_t)q->cfg.n_layers,
                        (uint32_t)p.tq, (uint32_t)p.to, (uint32_t)p.tf, (uint32_t)p.td,
                        (uint32_t)p.kb, (uint32_t)p.bm, (uint32_t)p.bn,
                        ((p.mode == MK_DECODE && p.fuse_combine == 1) ? 1u : 0u) | (p.loop ? 2u : 0u) |
                            ((p.mode == MK_DECODE && p.fuse_combine == 2) ? 4u : 0u) | (p.attn_pop ? 8u : 0u)};
      std::memcpy(d, h, sizeof(h));
      if (!q->segments.empty()) std::memcpy(d + 80, q->segments.data(), 16 * q->segments.size());
      break;
    }
    case MK_PART_INSTR: if (need) std::memcpy(d, q->instr.data(), need); break;
    case MK_PART_WAITS: if (need) std::memcpy(d, q->waits.data(), need); break;
    case MK_PART_TARGETS: if (need) std::memcpy(d, q->targets.data(), need); break;
    case MK_PART_DEVICE:
      std::memset(d, 0, need);
      if (!q->instr.empty()) std::memcpy(d + q->dev_instr_off, q->instr.data(), q->instr.size() * sizeof(mk::Instr));
      if (!q->waits.empty()) std::memcpy(d + q->dev_waits_off, q->waits.data(), q->waits.size() * sizeof(mk::Range));
      if (!q->targets.empty()) std::memcpy(d + q->dev_targets_off, q->targets.data(), q->targets.size() * 4);
      break;
  }
  return MK_OK;
}

void mk_queue_free(mk_queue* q) {
  if (!q) return;
  mk::forget_graphs(q->serial);
  delete q;
}

const char* mk_last_error(void) { return mk::last_error(); }

const char* mk_status_str(mk_status s) {
  switch (s) {
    case MK_OK: return "ok";
    case MK_EINVAL: return "invalid argument";
    case MK_ENOMEM: return "out of host memory";
    case MK_ELAUNCH: return "launch failed";
    case MK_EDEVICE: return "device error";
    case MK_ENOTSUP: return "not supported";
    default: return "unknown status";
  }
}

}  // extern "C"
