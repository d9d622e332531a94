// C ABI of the tile-synchronized decoder: argument checks, workspace layout,
// and the launches of one decode step (megakernel or one kernel per op).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <vector>

#include "kernels.h"
#include "mk.h"
#include "queue.h"

namespace mkd {
#define MK_DECL(T) Table table_##T##_1(); Table table_##T##_2(); Table table_##T##_4(); \
  Table table_##T##_8(); Table table_##T##_16(); Table table_##T##_32();
MK_DECL(bf16)
MK_DECL(f32)
#undef MK_DECL
Table table_prefill();
}  // namespace mkd

namespace {

using namespace mkd;

// ----------------------------------------------------------------------------- kernels used only here

__global__ void reset_kernel(uint32_t* counters, uint32_t n, uint32_t* heads, uint32_t nh, uint32_t* err) {
  const uint32_t stride = gridDim.x * blockDim.x;
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  for (uint32_t k = i; k < n; k += stride) counters[k] = 0;
  for (uint32_t k = i; k < nh * 32; k += stride) heads[k] = 0;
  for (uint32_t k = i; k < 8; k += stride) err[k] = 0;
}

__global__ void copy_rows_kernel(float* dst, const float* src, size_t n) {
  for (size_t k = blockIdx.x * (size_t)blockDim.x + threadIdx.x; k < n; k += (size_t)gridDim.x * blockDim.x) dst[k] = src[k];
}

__global__ __launch_bounds__(NT) void argmax_kernel(Args args) {
  KArgs& a = kernel_args();
  __shared__ float bv[NT];
  __shared__ int bi[NT];
  const int b = blockIdx.x;
  float best = -INFINITY;
  int besti = 0x7FFFFFFF;
  for (int k = threadIdx.x; k < a.lm_blocks; k += NT) {
    const float v = a.lm_val[(size_t)b * a.lm_blocks + k];
    const int i = a.lm_idx[(size_t)b * a.lm_blocks + k];
    if (v > best || (v == best && i < besti)) { best = v; besti = i; }
  }
  bv[threadIdx.x] = best;
  bi[threadIdx.x] = besti;
  __syncthreads();
  for (int w = NT / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      const float v = bv[threadIdx.x + w];
      const int i = bi[threadIdx.x + w];
      if (v > bv[threadIdx.x] || (v == bv[threadIdx.x] && i < bi[threadIdx.x])) { bv[threadIdx.x] = v; bi[threadIdx.x] = i; }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) a.next[b] = bi[0];
}


// ----------------------------------------------------------------------------- host side

struct Options {
  int workers_per_cu = 1;
  uint32_t spin_limit = 1u << 22;
  unsigned long long* trace = nullptr;   // device buffer, 64 bytes per instruction
  size_t trace_bytes = 0;
  int gemv_pipe = 0;                     // 0, 1: pipelined issue; 2: compiler-ordered issue
  uint32_t delay_seed = 0;               // race check: seeded stalls before tile stores
  int streams = 2;                       // multi-stream mode: internal streams per device
  int megakernels = 1;                   // megakernel mode: launches per step, cut at layer boundaries
  uint32_t prefill_lo = 15;              // prefill GEMMs taking the lo parts of their activations
};
Options g_opt;

// One process-wide lock over the library's host state: the options, the
// kernels' shared-memory opt-ins and the graph cache.  Every entry point that
// reads or writes them holds it; launches are asynchronous, so it is held only
// while a call enqueues its work.
std::mutex g_mu;

int num_cus() {
  static int n = 0;
  static std::once_flag once;
  std::call_once(once, [] {
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      n = 0;
    if (n <= 0) n = 256;
  });
  return n;
}

inline size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  size_t X, QKV, OPART, ATT, HRES, ACT, LMV, LMI, CTR, HEADS, ERR, total;
  size_t LMY, LMS;                           // decode with an LM head: its rows as bf16 hi / lo, row scales
  size_t sX, sQKV, sOP, sATT, sHRES, sACT;   // per-layer strides in floats
  int lm_blocks;
  // prefill only: bf16 GEMM operands (hi and lo parts) and per-row sums of squares (after ERR)
  size_t XB, XSS, HB, HSS, ATTB, ACTB, XBL, HBL, ATTBL, ACTBL;
  size_t sXB, sXSS, sATTB, sACTB;            // per-layer strides in elements
};

Layout layout(const mk_queue* q) {
  const mk_config& c = q->cfg;
  const size_t M = q->plan.rows, L = c.n_layers, hd = c.head_dim, r = c.n_q_heads / c.n_kv_heads;
  const size_t NQKV = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * hd;
  const size_t NS = q->n_splits ? q->n_splits : 1;
  Layout o{};
  o.sX = up256(M * c.hidden * 4) / 4;
  o.sQKV = up256(M * NQKV * 4) / 4;
  o.sOP = up256(M * c.n_kv_heads * NS * (r * hd + 2 * r) * 4) / 4;
  o.sATT = up256(M * c.n_q_heads * hd * 4) / 4;
  o.sHRES = up256(M * c.hidden * 4) / 4;
  o.sACT = up256(M * c.ffn * 4) / 4;
  o.lm_blocks = c.has_lm_head ? (c.vocab + LM_ROWS - 1) / LM_ROWS : 1;
  size_t off = 0;
  o.X = off; off += (L + 1) * o.sX * 4;
  o.QKV = off; off += L * o.sQKV * 4;
  o.OPART = off; off += L * o.sOP * 4;
  o.ATT = off; off += L * o.sATT * 4;
  o.HRES = off; off += L * o.sHRES * 4;
  o.ACT = off; off += L * o.sACT * 4;
  o.LMV = off; off += up256(M * o.lm_blocks * 4);
  o.LMI = off; off += up256(M * o.lm_blocks * 4);
  o.CTR = off; off += up256(q->targets.size() * 4);
  // sub-queue heads, then (run-time split hand-out) one split counter per layer
  o.HEADS = off; off += up256((size_t)(q->plan.n_queues + (q->plan.attn_pop ? L : 0)) * 128);
  o.ERR = off; off += 256;
  if (q->plan.mode == MK_DECODE && c.has_lm_head) {
    o.LMY = off; off += up256(2 * M * c.hidden * 2);
    o.LMS = off; off += up256(M * 4);
  }
  if (q->plan.mode == MK_PREFILL) {
    // bf16 copies of the GEMM activation operands, written by their producer
    // tiles (with the consumer's RMSNorm gain folded in for X and HRES) as hi
    // and lo parts, and sums of squares of X / HRES rows per 128-column tile
    const size_t nss = (c.hidden + 127) / 128;
    o.sXB = up256(M * c.hidden * 2) / 2;
    o.sXSS = up256(M * nss * 4) / 4;
    o.sATTB = up256(M * c.n_q_heads * hd * 2) / 2;
    o.sACTB = up256(M * c.ffn * 2) / 2;
    o.XB = off; off += L * o.sXB * 2;
    o.XSS = off; off += L * o.sXSS * 4;
    o.HB = off; off += L * o.sXB * 2;
    o.HSS = off; off += L * o.sXSS * 4;
    o.ATTB = off; off += L * o.sATTB * 2;
    o.ACTB = off; off += L * o.sACTB * 2;
    o.XBL = off; off += L * o.sXB * 2;
    o.HBL = off; off += L * o.sXB * 2;
    o.ATTBL = off; off += L * o.sATTB * 2;
    o.ACTBL = off; off += L * o.sACTB * 2;
  }
  o.total = off;
  return o;
}

Table pick_table(int dtype, int nb) {
  const bool bf = dtype == MK_BF16;
  if (nb <= 1) return bf ? table_bf16_1() : table_f32_1();
  if (nb <= 2) return bf ? table_bf16_2() : table_f32_2();
  if (nb <= 4) return bf ? table_bf16_4() : table_f32_4();
  if (nb <= 8) return bf ? table_bf16_8() : table_f32_8();
  if (nb <= 16) return bf ? table_bf16_16() : table_f32_16();
  return bf ? table_bf16_32() : table_f32_32();
}

constexpr uint32_t kMaxLds = 160 * 1024;

int nb_bucket(int rows) {
  return rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : rows <= 8 ? 8 : rows <= 16 ? 16 : 32;
}

struct LdsLayout { uint32_t res, x, ring, uni, bytes; };

// Bytes of the prefill tile region: the largest of a single-matrix GEMM tile
// (three stages of a 128 x 64 activation tile as hi and lo parts and of a
// 128 x 64 weight tile, row statistics), the gate/up tile (two stages of the
// activation pair and of a 256 x 64 weight tile) and an attention tile over 64
// query rows (Q as hi and lo, two 64-key K blocks, a V^T block, scores, the
// probabilities as hi and lo, row statistics).
constexpr uint32_t kPrefillGemmBytes = 3 * (2 * 128 * 128 + 128 * 128) + (256 + 128) * 4;
constexpr uint32_t kPrefillGateUpBytes = 2 * (2 * 128 * 128 + 256 * 128) + (256 + 128) * 4;
constexpr uint32_t kPrefillAttnBytes = 2 * (2 * 64 * 128) + 2 * (2 * 64 * 128) + 128 * 64 * 2 + 64 * 64 * 4 +
                                       2 * 64 * 64 * 2 + 3 * 64 * 4;

// Dynamic shared memory of one workgroup, in floats: header (index, norm
// factors), GEMV results, residual rows, then one region shared by the weight
// ring plus GEMV input staging and the attention buffers.  Mirrors make_smem()
// in kernels.h.
LdsLayout lds_layout(const mk_config& c, const mk_plan& p) {
  LdsLayout o{};
  if (p.mode == MK_PREFILL) {
    // prefill tiles use the header and the tile region only
    o.ring = (std::max({kPrefillGemmBytes, kPrefillGateUpBytes, kPrefillAttnBytes}) + 255) & ~255u;
    o.uni = o.ring / 4;
    o.bytes = 4 * (16 + 32 + NWAVE * 32) + o.ring;
    return o;
  }
  const uint32_t nb = nb_bucket(p.rows);
  auto r4 = [](uint32_t n) { return (n + 3) & ~3u; };
  const uint32_t max_rows = std::max({p.tq, p.to, 2 * p.tf, p.td, LM_ROWS});
  o.res = r4(max_rows * nb);
  const uint32_t kmax = std::max({c.hidden, c.ffn, c.n_q_heads * c.head_dim});
  o.x = std::max<uint32_t>(std::min<uint32_t>(XBUF_MAX, nb * kmax), nb * 512);
  // keep the whole layout within one workgroup's shared memory: shrink the
  // input staging (it is consumed in chunks of nb * 512 floats)
  o.ring = NWAVE * ring_lines_for(nb) * 1024;
  const uint32_t fixed = 4 * (16 + 32 + NWAVE * 32 + 2 * o.res) + o.ring;
  const uint32_t room = fixed < kMaxLds ? (kMaxLds - fixed) / 4 : 0;
  // fused split combines: the O-projection stages all of its input rows at once
  // (whole 512-column iterations) followed by every split partial of the rows
  uint32_t fused_need = 0;
  if (p.fuse_combine == 1) {
    const uint32_t r = c.n_q_heads / c.n_kv_heads, NA = c.n_q_heads * c.head_dim;
    const uint32_t NS = (p.ctx_max + p.kb - 1) / p.kb;
    fused_need = nb * ((NA + 511) / 512 * 512) + p.rows * c.n_kv_heads * NS * (r * c.head_dim + 2 * r) +
                 p.rows * c.n_kv_heads * r * NS;           // rows, partials, merge weights
    o.x = std::max(o.x, fused_need);
  }
  if (o.x > room) o.x = std::max<uint32_t>(room / (nb * 512) * (nb * 512), nb * 512);
  o.x = r4(o.x);
  const uint32_t r = c.n_q_heads / c.n_kv_heads, hd = c.head_dim;
  const uint32_t att = r4(r * hd) + 2 * r4(hd) + 2 * r4(hd / 2) + 2 * r4(NWAVE * ATT_MAX_R) + r4(NWAVE * r * hd);
  o.uni = std::max(o.ring / 4 + o.x, att);
  // the matrix-core GEMV's staging (bf16 weights, batched rows), where it fits
  if (c.dtype == MK_BF16 && nb >= MK_GEMV_MFMA_MIN_NB) {
    const uint32_t need = gemv_mfma_floats(gemv_mfma_cc(1, nb), nb);
    if (4 * (16 + 32 + NWAVE * 32 + 2 * o.res + need) <= kMaxLds) o.uni = std::max(o.uni, need);
  }
  o.bytes = 4 * (16 + 32 + NWAVE * 32 + 2 * o.res + o.uni);
  if (o.x < fused_need) o.bytes = kMaxLds + 1;            // does not fit: refused by the callers
  return o;
}
LdsLayout lds_layout(const mk_queue* q) { return lds_layout(q->cfg, q->plan); }

// Everything the kernels need except the per-call inputs and outputs.
void fill_args(const mk_queue* q, const void* d_queue, const mk_weights* w, const mk_kv* kv, void* d_workspace,
               const Layout& o, Args& a) {
  const mk_config& c = q->cfg;
  uint8_t* ws = static_cast<uint8_t*>(d_workspace);
  const uint8_t* qd = static_cast<const uint8_t*>(d_queue);
  a.L = c.n_layers; a.H = c.hidden; a.nq = c.n_q_heads; a.nkv = c.n_kv_heads; a.hd = c.head_dim;
  a.r = c.n_q_heads / c.n_kv_heads; a.F = c.ffn; a.V = c.vocab;
  a.NQKV = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim; a.NA = c.n_q_heads * c.head_dim;
  a.M = q->plan.rows; a.NS = q->n_splits; a.kb = q->plan.kb; a.ctx_max = q->plan.ctx_max;
  a.qk_norm = c.qk_norm; a.has_embed = c.has_embed; a.eps = c.rms_eps; a.theta = c.rope_theta;
  for (int i = 0; i < c.head_dim / 2 && i < 64; ++i)
    a.rope_inv[i] = std::pow((double)c.rope_theta, -2.0 * i / (double)c.head_dim);
  a.wqkv = w->wqkv; a.wo = w->wo; a.wgate = w->wgate; a.wup = w->wup; a.wdown = w->wdown;
  a.attn_norm = w->attn_norm; a.ffn_norm = w->ffn_norm; a.q_norm = w->q_norm; a.k_norm = w->k_norm;
  a.embed = w->embed; a.lm_head = w->lm_head; a.final_norm = w->final_norm;
  a.kc = kv->k; a.vc = kv->v;
  a.X = reinterpret_cast<float*>(ws + o.X); a.QKV = reinterpret_cast<float*>(ws + o.QKV);
  a.OPART = reinterpret_cast<float*>(ws + o.OPART); a.ATT = reinterpret_cast<float*>(ws + o.ATT);
  a.HRES = reinterpret_cast<float*>(ws + o.HRES); a.ACT = reinterpret_cast<float*>(ws + o.ACT);
  a.sX = o.sX; a.sQKV = o.sQKV; a.sOP = o.sOP; a.sATT = o.sATT; a.sHRES = o.sHRES; a.sACT = o.sACT;
  a.lm_val = reinterpret_cast<float*>(ws + o.LMV); a.lm_idx = reinterpret_cast<int*>(ws + o.LMI);
  a.lm_blocks = o.lm_blocks;
  a.lm_y = o.LMY ? reinterpret_cast<uint16_t*>(ws + o.LMY) : nullptr;
  a.lm_rs = o.LMS ? reinterpret_cast<float*>(ws + o.LMS) : nullptr;
  if (q->plan.mode == MK_PREFILL) {
    a.XB = reinterpret_cast<uint16_t*>(ws + o.XB); a.XSS = reinterpret_cast<float*>(ws + o.XSS);
    a.HB = reinterpret_cast<uint16_t*>(ws + o.HB); a.HSS = reinterpret_cast<float*>(ws + o.HSS);
    a.ATTB = reinterpret_cast<uint16_t*>(ws + o.ATTB); a.ACTB = reinterpret_cast<uint16_t*>(ws + o.ACTB);
    a.XBL = reinterpret_cast<uint16_t*>(ws + o.XBL); a.HBL = reinterpret_cast<uint16_t*>(ws + o.HBL);
    a.ATTBL = reinterpret_cast<uint16_t*>(ws + o.ATTBL); a.ACTBL = reinterpret_cast<uint16_t*>(ws + o.ACTBL);
    a.sXB = o.sXB; a.sXSS = o.sXSS; a.sATTB = o.sATTB; a.sACTB = o.sACTB;
  }
  a.counters = reinterpret_cast<uint32_t*>(ws + o.CTR); a.heads = reinterpret_cast<uint32_t*>(ws + o.HEADS);
  a.err = reinterpret_cast<uint32_t*>(ws + o.ERR);
  a.instr = reinterpret_cast<const Instr*>(qd + q->dev_instr_off);
  a.ranges = reinterpret_cast<const Range*>(qd + q->dev_waits_off);
  a.targets = reinterpret_cast<const uint32_t*>(qd + q->dev_targets_off);
  a.n_instr = (uint32_t)q->instr.size(); a.n_barriers = (uint32_t)q->targets.size();
  a.n_queues = (uint32_t)q->plan.n_queues;
  a.fuse_combine = q->plan.mode == MK_DECODE && q->plan.fuse_combine == 1;
  a.merge_last = q->plan.mode == MK_DECODE && q->plan.fuse_combine == 2;
  // run-time split hand-out: the layers' attention segments, of equal size and
  // evenly spaced (as the decode builder lays them out); else the static order
  a.attn_pop = 0;
  if (q->plan.mode == MK_DECODE && q->plan.attn_pop) {
    std::vector<const mk::Segment*> at;
    for (const mk::Segment& sg : q->segments)
      if (sg.op == mk::OP_ATTN) at.push_back(&sg);
    bool ok = !at.empty() && at.size() == (size_t)c.n_layers;
    const uint32_t stride = at.size() > 1 ? at[1]->first - at[0]->first : 0;
    for (size_t l = 0; ok && l < at.size(); ++l)
      ok = at[l]->layer == l && at[l]->count == at[0]->count && at[l]->first == at[0]->first + l * stride;
    if (ok) {
      a.attn_pop = 1;
      a.attn_first = at[0]->first; a.attn_stride = stride; a.attn_count = at[0]->count;
    }
  }
  a.range_begin = 0; a.range_end = (uint32_t)q->instr.size();
  const LdsLayout ll = lds_layout(q);
  a.lds_res = ll.res; a.lds_x = ll.x; a.lds_union = ll.uni; a.lds_bytes = ll.bytes; a.lds_ring = ll.ring;
  a.M_cache = kv && kv->rows > 0 ? kv->rows : q->plan.rows;
  a.lm_x = a.X + (size_t)c.n_layers * a.sX;
}

// Final RMSNorm + LM head GEMV (+ argmax) over the workspace's last hidden rows.
hipError_t launch_lm(const Table& t, const Args& a, bool want_next, hipStream_t stream) {
  // every buffer the LM-head kernels touch, and the staging offset past the ring
  if (!a.lm_x || !a.lm_head || !a.final_norm || !a.lm_val || !a.lm_idx || !a.lds_ring || a.M < 1)
    return hipErrorInvalidValue;
  hipError_t e = t.lm(a, stream);
  if (e == hipSuccess && want_next) {
    hipLaunchKernelGGL(argmax_kernel, dim3(a.M), dim3(NT), 0, stream, a);
    e = hipGetLastError();
  }
  return e;
}

#define FAIL(code, ...) do { mk::set_error(__VA_ARGS__); return (code); } while (0)

mk_status check_shapes(const mk_config& c) {
  if (c.hidden % 8 || c.ffn % 8 || (c.n_q_heads * c.head_dim) % 8)
    FAIL(MK_EINVAL, "hidden, ffn and n_q_heads*head_dim must be multiples of 8");
  if (c.head_dim != 64 && c.head_dim != 128) FAIL(MK_ENOTSUP, "head_dim must be 64 or 128");
  if (c.dtype == MK_F32 && c.head_dim != 64) FAIL(MK_ENOTSUP, "fp32 caches support head_dim 64 only");
  if (c.n_q_heads / c.n_kv_heads > ATT_MAX_R) FAIL(MK_ENOTSUP, "at most %d query heads per KV head", ATT_MAX_R);
  if (NT % ((c.n_q_heads / c.n_kv_heads) * c.head_dim / 8)) FAIL(MK_ENOTSUP, "query heads per KV head must be a power of two");
  if (c.dtype != MK_F32 && c.dtype != MK_BF16) FAIL(MK_EINVAL, "unknown dtype");
  return MK_OK;
}

// A refusal from the preparation step, as a status.
mk_status prep_status(hipError_t e) {
  if (e == hipSuccess) return MK_OK;
  if (e == hipErrorCooperativeLaunchTooLarge)
    FAIL(MK_ENOTSUP, "%d megakernel workgroups per compute unit do not fit its registers / shared memory",
         g_opt.workers_per_cu);
  FAIL(MK_ELAUNCH, "kernel set-up failed: %s", hipGetErrorString(e));
}

// ----------------------------------------------------------------------------- multi-stream mode

// MK_MULTI_STREAM: the step's (layer, op) segments go round-robin to S
// internal streams of the device (default priority, created on first use and
// kept for the process).  A fork event on the caller's stream, after the
// counter reset, starts them; the caller's stream waits on a join event of
// each before the LM head.  Segment k + 1 runs while segment k still does and
// waits on its tiles through the barrier counters.
//
// Progress: a stream runs one kernel at a time, so at most S segment kernels
// are active.  Each gets G = 8 * floor(per_cu * (CUs / 8) / S) workgroups (a
// multiple of the 8 XCDs, among which a dispatch's workgroups are spread
// evenly), and each kernel fits per_cu workgroups on a compute unit, so the
// active kernels' workgroups are resident together.  Every wait is on a
// segment enqueued earlier, which is active or done: no workgroup waits on one
// that cannot be scheduled.
constexpr int kMaxStreams = 8;
constexpr int kMaxMegakernels = 8;

// First instruction of layer l's ops (past the embedding tiles) in a decode queue.
uint32_t layer_first(const mk_queue* q, int l) {
  for (const mk::Segment& sg : q->segments)
    if ((int)sg.layer == l && sg.op != mk::OP_EMBED) return sg.first;
  return (uint32_t)q->instr.size();
}
constexpr int kXcds = 8;
struct StreamSet {
  hipStream_t st[kMaxStreams] = {};
  hipEvent_t join[kMaxStreams] = {};
  hipEvent_t fork = nullptr;
};
StreamSet g_streams[kMaxDevices];

hipError_t stream_set(int dev, int n, StreamSet*& out) {
  StreamSet& ss = g_streams[dev];
  hipError_t e = hipSuccess;
  if (!ss.fork) e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming);
  for (int i = 0; i < n && e == hipSuccess; ++i) {
    if (!ss.st[i]) e = hipStreamCreateWithFlags(&ss.st[i], hipStreamNonBlocking);
    if (e == hipSuccess && !ss.join[i]) e = hipEventCreateWithFlags(&ss.join[i], hipEventDisableTiming);
  }
  out = &ss;
  return e;
}

int ms_grid(int streams) {
  return kXcds * ((g_opt.workers_per_cu * (num_cus() / kXcds)) / streams);
}

hipError_t enqueue_multi_stream(const mk_queue* q, const Args& a, const Table& t, StreamSet& ss, int n,
                                hipStream_t stream) {
  const uint32_t grid = (uint32_t)ms_grid(n);
  hipError_t e = hipEventRecord(ss.fork, stream);
  for (int i = 0; i < n && e == hipSuccess; ++i) e = hipStreamWaitEvent(ss.st[i], ss.fork, 0);
  size_t k = 0;
  for (const mk::Segment& sg : q->segments) {
    if (e != hipSuccess) break;
    e = t.ms(a, sg.op, sg.first, sg.count, std::min(grid, sg.count), ss.st[k++ % n]);
  }
  // join every stream, also after a failed launch, so the caller's stream never
  // runs ahead of work already enqueued
  for (int i = 0; i < n; ++i) {
    hipError_t ej = hipEventRecord(ss.join[i], ss.st[i]);
    if (ej == hipSuccess) ej = hipStreamWaitEvent(stream, ss.join[i], 0);
    if (e == hipSuccess) e = ej;
  }
  return e;
}

// The launches of one decode step on `stream`, after every check passed:
// input rows, then (megakernel) the counter / head / error reset and one
// interpreter launch, (multi-stream, `ss` set) the counter / error reset and
// the segments on the internal streams, or (per op) the error reset and one
// launch per segment; then the LM head and argmax.
hipError_t enqueue_decode(const mk_queue* q, const Args& a, const Table& t, int exec_mode, bool want_lm,
                          bool want_next, hipStream_t stream, StreamSet* ss = nullptr, int n_streams = 0) {
  if (!q->cfg.has_embed) {
    // without an embedding the input rows are copied into X_0 by the first launch
    const size_t n = (size_t)a.M * a.H;
    hipLaunchKernelGGL(copy_rows_kernel, dim3((unsigned)std::min<size_t>((n + 255) / 256, 1024)), dim3(256), 0,
                       stream, a.X, a.x0, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool mega = exec_mode == MK_MEGAKERNEL;
  // counters: the tile waits (megakernel, multi-stream) and the split arrivals
  // of a queue whose last split merges (every mode)
  // heads: the sub-queues' pop counters and the layers' split counters
  const uint32_t nr = mega || ss || a.merge_last ? a.n_barriers : 0;
  const uint32_t nh = mega ? a.n_queues + (a.attn_pop ? (uint32_t)a.L : 0) : 0;
  hipLaunchKernelGGL(reset_kernel, dim3((nr + 255) / 256 + 1), dim3(256), 0, stream, a.counters, nr, a.heads, nh,
                     a.err);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (mega && g_opt.megakernels > 1) {
    // a composition of megakernels: launch k runs the layers [k L / K, (k + 1) L / K)
    // (the embedding with the first); kernel order covers the waits across launches
    const int K = g_opt.megakernels, L = q->cfg.n_layers;
    for (int k = 0; k < K && e == hipSuccess; ++k) {
      Args ak = a;
      ak.range_begin = k == 0 ? 0u : layer_first(q, k * L / K);
      ak.range_end = k == K - 1 ? (uint32_t)q->instr.size() : layer_first(q, (k + 1) * L / K);
      e = t.mega(ak, num_cus() * g_opt.workers_per_cu, stream);
    }
  } else if (mega) {
    e = t.mega(a, num_cus() * g_opt.workers_per_cu, stream);
  } else if (ss) {
    e = enqueue_multi_stream(q, a, t, *ss, n_streams, stream);
  } else {
    for (const mk::Segment& sg : q->segments) {
      e = t.kpo(a, sg.op, sg.first, sg.count, stream);
      if (e != hipSuccess) break;
    }
  }
  if (e == hipSuccess && want_lm) e = launch_lm(t, a, want_next, stream);
  return e;
}

// ----------------------------------------------------------------------------- kernel-per-op HIP graphs

// MK_KERNEL_PER_OP_GRAPH: the per-op launches of a step are captured once per
// distinct set of call arguments (every pointer, the queue, the options the
// kernels read) into an instantiated HIP graph, which later calls with the same
// arguments replay on the caller's stream.  The kernels read token ids,
// context lengths and inputs from device memory at run time, so a replay sees
// their current values.  At most kMaxGraphs graphs are kept; evicting one (or
// freeing its queue) first waits for its last replay to finish.
constexpr size_t kMaxGraphs = 16;
struct GraphEntry {
  std::vector<uint64_t> key;
  hipGraphExec_t exec = nullptr;
  hipEvent_t done = nullptr;       // recorded after each replay
  uint64_t last_use = 0;
};
std::vector<GraphEntry> g_graphs;
uint64_t g_graph_clock = 0;
hipStream_t g_capture_stream[kMaxDevices] = {};

void drop_graph(GraphEntry& g) {
  // best effort: a failed wait or destroy leaves nothing the caller could act on
  if (g.done) { (void)hipEventSynchronize(g.done); (void)hipEventDestroy(g.done); }
  if (g.exec) (void)hipGraphExecDestroy(g.exec);
  g.exec = nullptr; g.done = nullptr;
}

template <typename T> uint64_t u64(T v) { return (uint64_t)(uintptr_t)v; }

std::vector<uint64_t> graph_key(const mk_queue* q, int dev, const void* d_queue, const mk_weights* w, const mk_kv* kv,
                                const int32_t* tok, const float* x0, const int32_t* ctx, const void* ws,
                                size_t ws_bytes, const float* logits, const int32_t* next, const Args& a) {
  return {q->serial, (uint64_t)dev, u64(d_queue), u64(w->wqkv), u64(w->wo), u64(w->wgate), u64(w->wup),
          u64(w->wdown), u64(w->attn_norm), u64(w->ffn_norm), u64(w->q_norm), u64(w->k_norm), u64(w->embed),
          u64(w->lm_head), u64(w->final_norm), u64(kv->k), u64(kv->v), (uint64_t)kv->rows, u64(tok), u64(x0),
          u64(ctx), u64(ws), (uint64_t)ws_bytes, u64(logits), u64(next), (uint64_t)a.gemv_pipe, u64(a.trace),
          (uint64_t)a.spin_limit, (uint64_t)a.delay_seed};
}

mk_status graph_step(const mk_queue* q, const Args& a, const Table& t, std::vector<uint64_t> key, bool want_lm,
                     bool want_next, hipStream_t stream) {
  GraphEntry* hit = nullptr;
  for (GraphEntry& g : g_graphs)
    if (g.key == key) { hit = &g; break; }
  if (!hit) {
    const int dev = (int)key[1];
    if (!g_capture_stream[dev]) {
      hipError_t e = hipStreamCreateWithFlags(&g_capture_stream[dev], hipStreamNonBlocking);
      if (e != hipSuccess) FAIL(MK_ELAUNCH, "capture stream: %s", hipGetErrorString(e));
    }
    hipStream_t cs = g_capture_stream[dev];
    hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) FAIL(MK_ELAUNCH, "begin capture: %s", hipGetErrorString(e));
    const hipError_t el = enqueue_decode(q, a, t, MK_KERNEL_PER_OP, want_lm, want_next, cs);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(cs, &graph);
    if (el != hipSuccess || e != hipSuccess) {
      if (graph) (void)hipGraphDestroy(graph);
      FAIL(MK_ELAUNCH, "capture of the per-op launches: %s", hipGetErrorString(el != hipSuccess ? el : e));
    }
    GraphEntry ne;
    ne.key = std::move(key);
    e = hipGraphInstantiate(&ne.exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ne.done, hipEventDisableTiming);
    if (e != hipSuccess) {
      drop_graph(ne);
      FAIL(MK_ELAUNCH, "graph instantiation: %s", hipGetErrorString(e));
    }
    if (g_graphs.size() >= kMaxGraphs) {
      auto lru = std::min_element(g_graphs.begin(), g_graphs.end(),
                                  [](const GraphEntry& x, const GraphEntry& y) { return x.last_use < y.last_use; });
      drop_graph(*lru);
      g_graphs.erase(lru);
    }
    g_graphs.push_back(std::move(ne));
    hit = &g_graphs.back();
  }
  hit->last_use = ++g_graph_clock;
  hipError_t e = hipGraphLaunch(hit->exec, stream);
  if (e == hipSuccess) e = hipEventRecord(hit->done, stream);
  if (e != hipSuccess) FAIL(MK_ELAUNCH, "graph launch: %s", hipGetErrorString(e));
  return MK_OK;
}

// The common body of a decode step into a given workspace.
mk_status decode_impl(const mk_queue* q, const void* d_queue, const mk_weights* w, const mk_kv* kv,
                      const int32_t* d_tokens, const float* d_x0, const int32_t* d_ctx_lens, int32_t batch,
                      void* d_workspace, size_t workspace_nbytes, float* d_logits, int32_t* d_next,
                      int32_t exec_mode, hipStream_t stream) {
  if (!q || !d_queue || !w || !kv || !d_ctx_lens || !d_workspace) FAIL(MK_EINVAL, "null argument");
  if (q->plan.mode != MK_DECODE) FAIL(MK_EINVAL, "queue was not built for decode");
  if (q->plan.loop) FAIL(MK_EINVAL, "a loop queue runs through mk_decode_loop");
  const mk_config& c = q->cfg;
  if (mk_status st = check_shapes(c)) return st;
  if (batch != q->plan.rows) FAIL(MK_EINVAL, "batch %d differs from the queue's rows %d", batch, q->plan.rows);
  if (exec_mode != MK_MEGAKERNEL && exec_mode != MK_KERNEL_PER_OP && exec_mode != MK_KERNEL_PER_OP_GRAPH &&
      exec_mode != MK_MULTI_STREAM)
    FAIL(MK_EINVAL, "unknown exec_mode");
  if (lds_layout(q).bytes > kMaxLds) FAIL(MK_ENOTSUP, "tiles need more shared memory than a workgroup has");
  const Layout o = layout(q);
  if (workspace_nbytes < o.total) FAIL(MK_EINVAL, "workspace of %zu bytes, need %zu", workspace_nbytes, o.total);
  if (c.has_embed ? (!d_tokens || !w->embed) : !d_x0) FAIL(MK_EINVAL, "missing input tokens / rows");
  if (!w->wqkv || !w->wo || !w->wgate || !w->wup || !w->wdown || !w->attn_norm || !w->ffn_norm || !kv->k || !kv->v)
    FAIL(MK_EINVAL, "missing weights or cache");
  if (c.qk_norm && (!w->q_norm || !w->k_norm)) FAIL(MK_EINVAL, "missing QK-norm gains");
  if (c.has_lm_head && (d_logits || d_next) && (!w->lm_head || !w->final_norm)) FAIL(MK_EINVAL, "missing LM head");
  if (kv->rows != 0 && kv->rows != q->plan.rows) FAIL(MK_EINVAL, "decode cache rows must equal the batch");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) FAIL(MK_ELAUNCH, "no current device");
  if (exec_mode == MK_MEGAKERNEL && num_cus() * g_opt.workers_per_cu < q->plan.n_queues)
    FAIL(MK_EINVAL, "fewer workers than sub-queues");
  if (exec_mode == MK_MEGAKERNEL && g_opt.megakernels > 1) {
    if (num_cus() * g_opt.workers_per_cu != q->plan.n_queues)
      FAIL(MK_ENOTSUP, "a composition of megakernels needs one sub-queue per worker");
    if (g_opt.megakernels > c.n_layers) FAIL(MK_ENOTSUP, "more megakernels than layers");
  }

  Args a{};
  fill_args(q, d_queue, w, kv, d_workspace, o, a);
  a.tokens = d_tokens; a.x0 = d_x0; a.ctx_lens = d_ctx_lens;
  a.logits = d_logits; a.next = d_next;
  a.spin_limit = g_opt.spin_limit;
  a.gemv_pipe = g_opt.gemv_pipe;
  a.delay_seed = g_opt.delay_seed;
  a.trace = (g_opt.trace && g_opt.trace_bytes >= 64 * q->instr.size()) ? g_opt.trace : nullptr;

  const Table t = pick_table(c.dtype, a.M);
  const bool want_lm = c.has_lm_head && (d_logits || d_next);
  const int prep_mode = exec_mode == MK_MEGAKERNEL ? MK_MEGAKERNEL
                        : exec_mode == MK_MULTI_STREAM ? kMultiStreamMode : MK_KERNEL_PER_OP;
  hipError_t e = t.prep(a, prep_mode, g_opt.workers_per_cu);
  if (e == hipSuccess && want_lm) e = t.prep_lm(a);
  if (mk_status st = prep_status(e)) return st;
  if (exec_mode == MK_MULTI_STREAM) {
    if (ms_grid(g_opt.streams) < 1) FAIL(MK_ENOTSUP, "%d streams leave no workgroups per kernel", g_opt.streams);
    StreamSet* ss = nullptr;
    e = stream_set(dev, g_opt.streams, ss);
    if (e != hipSuccess) FAIL(MK_ELAUNCH, "internal streams: %s", hipGetErrorString(e));
    e = enqueue_decode(q, a, t, exec_mode, want_lm, d_next != nullptr, stream, ss, g_opt.streams);
    if (e != hipSuccess) FAIL(MK_ELAUNCH, "launch failed: %s", hipGetErrorString(e));
    return MK_OK;
  }
  if (exec_mode == MK_KERNEL_PER_OP_GRAPH)
    return graph_step(q, a, t,
                      graph_key(q, dev, d_queue, w, kv, d_tokens, d_x0, d_ctx_lens, d_workspace, workspace_nbytes,
                                d_logits, d_next, a),
                      want_lm, d_next != nullptr, stream);
  e = enqueue_decode(q, a, t, exec_mode, want_lm, d_next != nullptr, stream);
  if (e != hipSuccess) FAIL(MK_ELAUNCH, "launch failed: %s", hipGetErrorString(e));
  return MK_OK;
}

// ----------------------------------------------------------------------------- static scratch

// The workspace of mk_decode_step_static: a file-scope device array, one copy
// per device the library runs on, held until the process ends.  Host code never
// uses the array's name as an address (on the host it is only a stand-in): the
// device address comes from hipGetSymbolAddress, once per device, with that
// device current.
constexpr size_t kScratchBytes = size_t(64) << 20;
void* g_scratch[kMaxDevices] = {};

__global__ void copy_words_kernel(uint32_t* dst, const uint32_t* src, uint32_t n) {
  if (threadIdx.x < n) dst[threadIdx.x] = src[threadIdx.x];
}

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
mk_status scratch_of_device(int dev, void** out) {
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) FAIL(MK_ELAUNCH, "address of the static scratch: %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MK_OK;
}
}  // namespace

namespace mk {
// Called by mk_queue_free: the graphs captured for a queue die with it.
void forget_graphs(uint64_t serial) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (size_t i = 0; i < g_graphs.size();) {
    if (g_graphs[i].key[0] == serial) {
      drop_graph(g_graphs[i]);
      g_graphs.erase(g_graphs.begin() + i);
    } else {
      ++i;
    }
  }
}
}  // namespace mk

extern "C" {

mk_status mk_workspace_nbytes(const mk_queue* q, size_t* nbytes) {
  if (!q || !nbytes) FAIL(MK_EINVAL, "null argument");
  *nbytes = layout(q).total;
  return MK_OK;
}

mk_status mk_workspace_offset(const mk_queue* q, int32_t tensor, int32_t layer, size_t* offset) {
  if (!q || !offset) FAIL(MK_EINVAL, "null argument");
  const Layout o = layout(q);
  const int L = q->cfg.n_layers;
  const int lmax = tensor == MK_T_X ? L : (tensor <= MK_T_ACT ? L - 1 : 0);
  if (layer < 0 || layer > lmax) FAIL(MK_EINVAL, "layer %d out of range for tensor %d", layer, tensor);
  switch (tensor) {
    case MK_T_X: *offset = o.X + (size_t)layer * o.sX * 4; break;
    case MK_T_QKV: *offset = o.QKV + (size_t)layer * o.sQKV * 4; break;
    case MK_T_OPART: *offset = o.OPART + (size_t)layer * o.sOP * 4; break;
    case MK_T_ATT: *offset = o.ATT + (size_t)layer * o.sATT * 4; break;
    case MK_T_HRES: *offset = o.HRES + (size_t)layer * o.sHRES * 4; break;
    case MK_T_ACT: *offset = o.ACT + (size_t)layer * o.sACT * 4; break;
    case MK_T_COUNTERS: *offset = o.CTR; break;
    case MK_T_HEADS: *offset = o.HEADS; break;
    case MK_T_ERROR: *offset = o.ERR; break;
    case MK_T_LMPART: *offset = o.LMV; break;
    default: FAIL(MK_EINVAL, "unknown tensor %d", tensor);
  }
  return MK_OK;
}

mk_status mk_decode_step(const mk_queue* q, const void* d_queue, const mk_weights* w, const mk_kv* kv,
                         const int32_t* d_tokens, const float* d_x0, const int32_t* d_ctx_lens,
                         int32_t batch, void* d_workspace, size_t workspace_nbytes, float* d_logits,
                         int32_t* d_next, int32_t exec_mode, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_mu);
  return decode_impl(q, d_queue, w, kv, d_tokens, d_x0, d_ctx_lens, batch, d_workspace, workspace_nbytes, d_logits,
                     d_next, exec_mode, stream);
}

mk_status mk_decode_step_static(const mk_queue* q, const void* d_queue, const mk_weights* w, const mk_kv* kv,
                                const int32_t* d_tokens, const float* d_x0, const int32_t* d_ctx_lens,
                                int32_t batch, float* d_logits, int32_t* d_next, uint32_t* d_error,
                                int32_t exec_mode, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!q) FAIL(MK_EINVAL, "null argument");
  if (exec_mode == MK_KERNEL_PER_OP_GRAPH || exec_mode == MK_MULTI_STREAM)
    FAIL(MK_EINVAL, "the static-scratch step has no graph or multi-stream mode (graphs and streams allocate)");
  const size_t need = layout(q).total;
  if (need > kScratchBytes)
    FAIL(MK_EINVAL, "the step needs %zu bytes of workspace; the static scratch holds %zu", need, kScratchBytes);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) FAIL(MK_ELAUNCH, "no current device");
  void* ws = nullptr;
  if (mk_status st = scratch_of_device(dev, &ws)) return st;
  if (mk_status st = decode_impl(q, d_queue, w, kv, d_tokens, d_x0, d_ctx_lens, batch, ws, kScratchBytes,
                                 d_logits, d_next, exec_mode, stream))
    return st;
  if (d_error) {
    hipLaunchKernelGGL(copy_words_kernel, dim3(1), dim3(64), 0, stream, d_error,
                       reinterpret_cast<const uint32_t*>(static_cast<uint8_t*>(ws) + layout(q).ERR), 8u);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) FAIL(MK_ELAUNCH, "copy of the error record: %s", hipGetErrorString(e));
  }
  return MK_OK;
}

mk_status mk_decode_loop(const mk_queue* q, const void* d_queue, const mk_weights* w, const mk_kv* kv,
                         const int32_t* d_tokens, const int32_t* d_ctx_lens, int32_t batch, int32_t steps,
                         int32_t feedback, void* d_workspace, size_t workspace_nbytes, float* d_logits,
                         int32_t* d_next, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!q || !d_queue || !w || !kv || !d_tokens || !d_ctx_lens || !d_workspace || !d_next)
    FAIL(MK_EINVAL, "null argument");
  if (q->plan.mode != MK_DECODE || !q->plan.loop) FAIL(MK_EINVAL, "the queue was not built as a loop queue");
  const mk_config& c = q->cfg;
  if (mk_status st = check_shapes(c)) return st;
  if (c.dtype != MK_BF16) FAIL(MK_ENOTSUP, "multi-step decode is built for bf16 models");
  if (batch != q->plan.rows) FAIL(MK_EINVAL, "batch %d differs from the queue's rows %d", batch, q->plan.rows);
  if (steps < 1) FAIL(MK_EINVAL, "steps must be positive");
  if (feedback != 0 && feedback != 1) FAIL(MK_EINVAL, "feedback must be 0 or 1");
  if ((uint64_t)steps * q->instr.size() > 0xFFFFFFFEull) FAIL(MK_EINVAL, "too many steps for one launch");
  if (lds_layout(q).bytes > kMaxLds) FAIL(MK_ENOTSUP, "tiles need more shared memory than a workgroup has");
  const Layout o = layout(q);
  if (workspace_nbytes < o.total) FAIL(MK_EINVAL, "workspace of %zu bytes, need %zu", workspace_nbytes, o.total);
  if (!w->wqkv || !w->wo || !w->wgate || !w->wup || !w->wdown || !w->attn_norm || !w->ffn_norm || !w->embed ||
      !w->lm_head || !w->final_norm || !kv->k || !kv->v)
    FAIL(MK_EINVAL, "missing weights or cache");
  if (c.qk_norm && (!w->q_norm || !w->k_norm)) FAIL(MK_EINVAL, "missing QK-norm gains");
  if (kv->rows != 0 && kv->rows != q->plan.rows) FAIL(MK_EINVAL, "decode cache rows must equal the batch");
  if (num_cus() * g_opt.workers_per_cu < q->plan.n_queues) FAIL(MK_EINVAL, "fewer workers than sub-queues");

  Args a{};
  fill_args(q, d_queue, w, kv, d_workspace, o, a);
  a.tokens = d_tokens; a.ctx_lens = d_ctx_lens;
  a.logits = d_logits; a.next = nullptr; a.next_all = d_next;
  a.steps = steps; a.feedback = feedback;
  a.spin_limit = g_opt.spin_limit;
  a.gemv_pipe = g_opt.gemv_pipe;
  a.delay_seed = g_opt.delay_seed;
  a.trace = (g_opt.trace && g_opt.trace_bytes >= 64 * q->instr.size()) ? g_opt.trace : nullptr;
  const Table t = pick_table(c.dtype, a.M);
  if (!t.loop) FAIL(MK_ENOTSUP, "no multi-step interpreter for this model");
  if (mk_status st = prep_status(t.prep(a, kLoopMode, g_opt.workers_per_cu))) return st;
  hipLaunchKernelGGL(reset_kernel, dim3((a.n_barriers + 255) / 256 + 1), dim3(256), 0, stream, a.counters,
                     a.n_barriers, a.heads, a.n_queues, a.err);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = t.loop(a, num_cus() * g_opt.workers_per_cu, stream);
  if (e != hipSuccess) FAIL(MK_ELAUNCH, "launch failed: %s", hipGetErrorString(e));
  return MK_OK;
}

mk_status mk_lm_head(const mk_queue* q, const mk_weights* w, void* d_workspace, size_t workspace_nbytes,
                     float* d_logits, int32_t* d_next, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!q || !w || !d_workspace) FAIL(MK_EINVAL, "null argument");
  const mk_config& c = q->cfg;
  if (!c.has_lm_head) FAIL(MK_EINVAL, "the model has no LM head");
  if (!w->lm_head || !w->final_norm) FAIL(MK_EINVAL, "missing LM head");
  if (!d_logits && !d_next) return MK_OK;
  if (q->plan.mode != MK_DECODE) FAIL(MK_EINVAL, "queue was not built for decode");
  const Layout o = layout(q);
  if (workspace_nbytes < o.total) FAIL(MK_EINVAL, "workspace of %zu bytes, need %zu", workspace_nbytes, o.total);
  Args a{};
  uint8_t* ws = static_cast<uint8_t*>(d_workspace);
  a.L = c.n_layers; a.H = c.hidden; a.V = c.vocab; a.M = q->plan.rows;
  a.eps = c.rms_eps;
  a.lm_head = w->lm_head; a.final_norm = w->final_norm;
  a.X = reinterpret_cast<float*>(ws + o.X); a.sX = o.sX;
  a.lm_val = reinterpret_cast<float*>(ws + o.LMV); a.lm_idx = reinterpret_cast<int*>(ws + o.LMI);
  a.lm_blocks = o.lm_blocks; a.err = reinterpret_cast<uint32_t*>(ws + o.ERR);
  a.lm_y = o.LMY ? reinterpret_cast<uint16_t*>(ws + o.LMY) : nullptr;
  a.lm_rs = o.LMS ? reinterpret_cast<float*>(ws + o.LMS) : nullptr;
  a.r = c.n_q_heads / c.n_kv_heads; a.hd = c.head_dim;
  a.lm_x = a.X + (size_t)c.n_layers * a.sX;
  const LdsLayout ll = lds_layout(q);
  a.lds_res = ll.res; a.lds_x = ll.x; a.lds_union = ll.uni; a.lds_bytes = ll.bytes; a.lds_ring = ll.ring;
  a.logits = d_logits; a.next = d_next;
  const Table t = pick_table(c.dtype, a.M);
  if (mk_status st = prep_status(t.prep_lm(a))) return st;
  const hipError_t e = launch_lm(t, a, d_next != nullptr, stream);
  if (e != hipSuccess) FAIL(MK_ELAUNCH, "launch failed: %s", hipGetErrorString(e));
  return MK_OK;
}

mk_status mk_prefill(const mk_queue* q, const void* d_queue, const mk_weights* w, const mk_kv* kv,
                     const int32_t* d_tokens, int32_t seq_len, int32_t kv_row, void* d_workspace,
                     size_t workspace_nbytes, float* d_logits_last, int32_t* d_next, int32_t exec_mode,
                     hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!q || !d_queue || !w || !kv || !d_tokens || !d_workspace) FAIL(MK_EINVAL, "null argument");
  if (q->plan.mode != MK_PREFILL) FAIL(MK_EINVAL, "queue was not built for prefill");
  const mk_config& c = q->cfg;
  if (mk_status st = check_shapes(c)) return st;
  if (c.dtype != MK_BF16 || !c.has_embed) FAIL(MK_ENOTSUP, "prefill needs a bf16 model with an embedding");
  if (c.head_dim != 128 || q->plan.bm != 128 || q->plan.bn != 128)
    FAIL(MK_ENOTSUP, "prefill tiles are 128 x 128 over 128-wide heads");
  if (c.hidden % 128 || c.ffn % 64 || (c.n_q_heads * c.head_dim) % 64)
    FAIL(MK_ENOTSUP, "prefill needs the hidden size a multiple of 128 and the other K dimensions of 64");
  if (seq_len < 1 || seq_len > q->plan.rows) FAIL(MK_EINVAL, "seq_len %d outside 1..%d", seq_len, q->plan.rows);
  if (kv->rows < 1 || kv_row < 0 || kv_row >= kv->rows) FAIL(MK_EINVAL, "kv_row outside the cache rows");
  if (exec_mode != MK_MEGAKERNEL && exec_mode != MK_KERNEL_PER_OP) FAIL(MK_EINVAL, "unknown exec_mode");
  if (lds_layout(q).bytes > kMaxLds) FAIL(MK_ENOTSUP, "tiles need more shared memory than a workgroup has");
  const Layout o = layout(q);
  if (workspace_nbytes < o.total) FAIL(MK_EINVAL, "workspace of %zu bytes, need %zu", workspace_nbytes, o.total);
  if (!w->wqkv || !w->wo || !w->wgate || !w->wup || !w->wdown || !w->attn_norm || !w->ffn_norm || !w->embed ||
      !kv->k || !kv->v)
    FAIL(MK_EINVAL, "missing weights or cache");
  if (c.qk_norm && (!w->q_norm || !w->k_norm)) FAIL(MK_EINVAL, "missing QK-norm gains");
  if ((d_logits_last || d_next) && (!c.has_lm_head || !w->lm_head || !w->final_norm)) FAIL(MK_EINVAL, "missing LM head");
  if (exec_mode == MK_MEGAKERNEL && num_cus() * g_opt.workers_per_cu < q->plan.n_queues)
    FAIL(MK_EINVAL, "fewer workers than sub-queues");

  Args a{};
  fill_args(q, d_queue, w, kv, d_workspace, o, a);
  a.tokens = d_tokens; a.seq_len = seq_len; a.kv_row = kv_row; a.M_cache = kv->rows;
  a.prefill_lo = g_opt.prefill_lo;
  a.spin_limit = g_opt.spin_limit;
  a.gemv_pipe = g_opt.gemv_pipe;
  a.delay_seed = g_opt.delay_seed;
  a.trace = (g_opt.trace && g_opt.trace_bytes >= 64 * q->instr.size()) ? g_opt.trace : nullptr;
  // LM head on the last prompt position only, with the one-row decode layout
  const bool want_lm = d_logits_last || d_next;
  Args lm = a;
  if (want_lm) {
    lm.M = 1;
    mk_plan lp = q->plan;
    lp.mode = MK_DECODE; lp.rows = 1;
    const LdsLayout ll = lds_layout(c, lp);
    lm.lds_res = ll.res; lm.lds_x = ll.x; lm.lds_union = ll.uni; lm.lds_bytes = ll.bytes; lm.lds_ring = ll.ring;
    lm.lm_x = a.X + (size_t)c.n_layers * a.sX + (size_t)(seq_len - 1) * c.hidden;
    lm.logits = d_logits_last; lm.next = d_next;
  }
  const Table t = table_prefill();
  const Table tl = pick_table(c.dtype, 1);
  hipError_t e = t.prep(a, exec_mode, g_opt.workers_per_cu);
  if (e == hipSuccess && want_lm) e = tl.prep_lm(lm);
  if (mk_status st = prep_status(e)) return st;

  const bool mega = exec_mode == MK_MEGAKERNEL;
  const uint32_t nr = mega ? a.n_barriers : 0, nh = mega ? a.n_queues : 0;
  hipLaunchKernelGGL(reset_kernel, dim3((nr + 255) / 256 + 1), dim3(256), 0, stream, a.counters, nr, a.heads, nh,
                     a.err);
  e = hipGetLastError();
  if (e == hipSuccess) {
    if (mega) {
      e = t.mega(a, num_cus() * g_opt.workers_per_cu, stream);
    } else {
      for (const mk::Segment& sg : q->segments) {
        e = t.kpo(a, sg.op, sg.first, sg.count, stream);
        if (e != hipSuccess) break;
      }
    }
  }
  if (e == hipSuccess && want_lm) e = launch_lm(tl, lm, d_next != nullptr, stream);
  if (e != hipSuccess) FAIL(MK_ELAUNCH, "launch failed: %s", hipGetErrorString(e));
  return MK_OK;
}

mk_status mk_device_error(const mk_queue* q, const void* d_workspace, mk_dev_error* out, hipStream_t stream) {
  if (!q || !d_workspace || !out) FAIL(MK_EINVAL, "null argument");
  const Layout o = layout(q);
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) FAIL(MK_EDEVICE, "stream: %s", hipGetErrorString(e));
  uint32_t rec[8];
  e = hipMemcpy(rec, static_cast<const uint8_t*>(d_workspace) + o.ERR, sizeof(rec), hipMemcpyDeviceToHost);
  if (e != hipSuccess) FAIL(MK_EDEVICE, "copy: %s", hipGetErrorString(e));
  out->code = rec[0]; out->instr = rec[1]; out->barrier = rec[2]; out->value = rec[3]; out->target = rec[4];
  return rec[0] ? MK_EDEVICE : MK_OK;
}

mk_status mk_set_option(int32_t key, int64_t value) {
  std::lock_guard<std::mutex> lk(g_mu);
  switch (key) {
    case MK_OPT_WORKERS_PER_CU:
      if (value < 1 || value > 8) FAIL(MK_EINVAL, "workers per CU must be 1..8");
      g_opt.workers_per_cu = (int)value; return MK_OK;
    case MK_OPT_SPIN_LIMIT:
      if (value < 1 || value > (int64_t)1 << 31) FAIL(MK_EINVAL, "spin limit out of range");
      g_opt.spin_limit = (uint32_t)value; return MK_OK;
    case MK_OPT_TRACE_BUFFER:
      g_opt.trace = reinterpret_cast<unsigned long long*>(static_cast<uintptr_t>(value)); return MK_OK;
    case MK_OPT_TRACE_BYTES:
      if (value < 0) FAIL(MK_EINVAL, "negative trace size");
      g_opt.trace_bytes = (size_t)value; return MK_OK;
    case MK_OPT_GEMV_PIPE:
      if (value < 0 || value > 2) FAIL(MK_EINVAL, "GEMV issue mode must be 0, 1 or 2");
      g_opt.gemv_pipe = (int)value; return MK_OK;
    case MK_OPT_DELAY_SEED:
      if (value < 0 || value > 0xFFFFFFFFll) FAIL(MK_EINVAL, "delay seed must fit 32 bits");
      g_opt.delay_seed = (uint32_t)value; return MK_OK;
    case MK_OPT_STREAMS:
      if (value < 1 || value > kMaxStreams) FAIL(MK_EINVAL, "streams must be 1..%d", kMaxStreams);
      g_opt.streams = (int)value; return MK_OK;
    case MK_OPT_MEGAKERNELS:
      if (value < 1 || value > kMaxMegakernels) FAIL(MK_EINVAL, "megakernels must be 1..%d", kMaxMegakernels);
      g_opt.megakernels = (int)value; return MK_OK;
    case MK_OPT_PREFILL_LO:
      if (value < 0 || value > 15) FAIL(MK_EINVAL, "prefill lo-part mask must be 0..15");
      g_opt.prefill_lo = (uint32_t)value; return MK_OK;
    default: FAIL(MK_EINVAL, "unknown or read-only option %d", key);
  }
}

int64_t mk_get_option(int32_t key) {
  if (key == MK_OPT_NUM_CUS) return num_cus();
  std::lock_guard<std::mutex> lk(g_mu);
  switch (key) {
    case MK_OPT_WORKERS_PER_CU: return g_opt.workers_per_cu;
    case MK_OPT_SPIN_LIMIT: return g_opt.spin_limit;
    case MK_OPT_TRACE_BUFFER: return (int64_t)(uintptr_t)g_opt.trace;
    case MK_OPT_TRACE_BYTES: return (int64_t)g_opt.trace_bytes;
    case MK_OPT_GEMV_PIPE: return g_opt.gemv_pipe;
    case MK_OPT_DELAY_SEED: return g_opt.delay_seed;
    case MK_OPT_STREAMS: return g_opt.streams;
    case MK_OPT_MEGAKERNELS: return g_opt.megakernels;
    case MK_OPT_PREFILL_LO: return g_opt.prefill_lo;
    default: return -1;
  }
}

}  // extern "C"
