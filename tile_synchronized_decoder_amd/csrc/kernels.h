// Tile-synchronized decoder for gfx950: op bodies, the persistent interpreter,
// the kernel-per-operator kernels and the LM head (device code, templates).
//
// Method (sources cited in include/mk.h): one persistent kernel whose
// workgroups act as interpreters ("Production Megakernels" lecture summary,
// Technical details: a loop around a switch; cores atomically pop
// instructions from a global queue in DRAM).  Each instruction computes one
// tile of one intermediate tensor and first waits on the counters of exactly
// the producer tiles it reads (MegaOps abstract: tile-granular dependencies
// instead of kernel barriers), issuing its weight loads before it waits so the
// weights stream while producers finish (MegaOps abstract: prefetching
// weights while the preceding kernel runs; lecture summary: memory
// pipelining).  The decoder arithmetic is the standard pre-norm Llama/Qwen
// block.
//
// gfx950 specifics: 64-lane wavefronts, 4 waves (256 threads) per workgroup,
// one workgroup per compute unit by default; weights stream into shared
// memory by direct-to-LDS loads.  The tile hand-off does not use whole-cache
// release / acquire (on this part that writes back or invalidates every
// per-XCD L2): intermediate tiles are stored and loaded only with agent-scope
// (sc1) atomic accesses, which are coherent across the XCDs' L2 caches; a
// producer waits until its stores are acknowledged (vmcnt 0) before one
// thread bumps the tile's counter, and a consumer issues its tile loads only
// after its poll of the counter has returned.  See signal_tile / wait_tiles.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <algorithm>
#include <mutex>

#include "mk.h"
#include "queue.h"


namespace mkd {

using mk::Instr;
using mk::Range;

constexpr int NT = 256;                 // threads per workgroup
constexpr int NWAVE = NT / 64;
constexpr int XBUF_MAX = 36864;         // LDS staging of GEMV inputs, upper bound (144 KB)
constexpr int ROWS_PER_PASS_MAX = 16;   // GEMV rows reduced per pass (4 waves x 4)
constexpr int ATT_MAX_R = 4;            // query heads per KV head
constexpr int LM_ROWS = 64;             // vocabulary rows per LM-head workgroup
// Weight lines (1 KB) in flight per wave: 20 for one or two input rows (80 KB
// per workgroup; 16, 24, 28 and 32 measured slower for the 1B shape), 16 for
// more.  Batched GEMVs do more arithmetic per line and need the shared memory
// for their inputs, so their rings are shorter.
#ifndef MK_RING_LINES_SMALL
#define MK_RING_LINES_SMALL 20
#endif
// Smallest input-row bucket whose bf16 GEMVs run on the matrix cores (at one
// and two rows the vector units keep up with HBM).
#ifndef MK_GEMV_MFMA_MIN_NB
#define MK_GEMV_MFMA_MIN_NB 4
#endif
constexpr int ring_lines_for(int nb) { return nb <= 2 ? MK_RING_LINES_SMALL : 16; }
template <int NB> constexpr int ring_lines() { return ring_lines_for(NB); }
constexpr uint32_t ERR_TIMEOUT = 1, ERR_OPCODE = 2, ERR_CONTEXT = 3, ERR_TOKEN = 4;

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __bf16 dbf16x8 __attribute__((ext_vector_type(8)));    // a matrix-core operand fragment
typedef float df32x16 __attribute__((ext_vector_type(16)));    // a 32 x 32 accumulator fragment

// ----------------------------------------------------------------------------- kernel arguments

struct Args {
  // shape
  int L, H, nq, nkv, hd, r, F, V, NQKV, NA, M, NS, kb, ctx_max, qk_norm, has_embed;
  float eps;
  double theta;
  // weights
  const void* wqkv; const void* wo; const void* wgate; const void* wup; const void* wdown;
  const float* attn_norm; const float* ffn_norm; const float* q_norm; const float* k_norm;
  const void* embed; const void* lm_head; const float* final_norm;
  void* kc; void* vc;
  // workspace
  float* X; float* QKV; float* OPART; float* ATT; float* HRES; float* ACT;
  size_t sX, sQKV, sOP, sATT, sHRES, sACT;     // per-layer strides (floats)
  float* lm_val; int* lm_idx; int lm_blocks;
  uint32_t* counters; uint32_t* heads; uint32_t* err;
  // queue
  const Instr* instr; const Range* ranges; const uint32_t* targets;
  uint32_t n_instr, n_barriers, n_queues;
  // runtime inputs / outputs
  const int* tokens; const float* x0; const int* ctx_lens;
  float* logits; int* next;
  uint32_t spin_limit;
  // dynamic shared memory layout, in floats (see lds_layout on the host)
  uint32_t lds_res, lds_x, lds_union, lds_bytes;
  // rotary inverse frequencies theta^(-2i/hd), i < hd/2, computed in float64 on the host
  double rope_inv[64];
  // optional per-instruction trace: TRACE_WORDS x u64 per instruction (see mk.h)
  unsigned long long* trace;
  // prefill: runtime prompt length, cache row written, rows of the cache allocation
  int seq_len, kv_row, M_cache;
  uint32_t lds_ring;             // bytes of the ring / prefill tile region
  const float* lm_x;             // LM head input rows
  uint16_t* lm_y;                // [2][M][H]: the LM head's normalised rows as bf16 hi, lo (matrix-core head)
  float* lm_rs;                  // [M]: their RMSNorm scales
  int gemv_pipe;                 // decode GEMV weight issue: 0, 1 pipelined; 2 compiler-ordered
  uint32_t prefill_lo;           // prefill GEMMs taking their activations' lo parts (P_LO_* bits)
  int fuse_combine;              // decode queue without split combines: O-projection merges the partials
  int merge_last;                // decode queue without split combines: the last split to arrive merges
  // megakernel, one sub-queue per worker: a layer's attention splits (the
  // instructions attn_first + l * attn_stride + [0, attn_count)) are handed out
  // from the layer's counter heads[(n_queues + l) * 32]
  int attn_pop;
  uint32_t attn_first, attn_stride, attn_count;
  // megakernel (one sub-queue per worker, not loop queues): the launch runs the
  // queue positions [range_begin, range_end) (all of them, unless the step is
  // a composition of several megakernels cut at layer boundaries)
  uint32_t range_begin, range_end;
  uint32_t delay_seed;           // race check: seeded stall before each tile's stores (0: off)
  // persistent multi-step decode (loop queues): steps of the run, 1 = embed the
  // previous step's argmax (else tokens[step][row]), the argmax of every step
  // [steps][rows] (logits, when given, are [steps][rows][V])
  int steps, feedback;
  int* next_all;
  // prefill: bf16 GEMM operands (X and HRES with the consumer's RMSNorm gain
  // applied), each as a pair: hi = bf16(y) and lo = bf16(y - hi), per-row sums
  // of squares of X / HRES per 128-column tile
  uint16_t* XB; uint16_t* HB; uint16_t* ATTB; uint16_t* ACTB;
  uint16_t* XBL; uint16_t* HBL; uint16_t* ATTBL; uint16_t* ACTBL;
  float* XSS; float* HSS;
  size_t sXB, sXSS, sATTB, sACTB;              // per-layer strides (elements)
};

// Device code reads the arguments in place, through a constant-address-space
// reference to the kernel argument segment: loads stay scalar, and the
// interpreter launders the pointer every iteration so the compiler cannot
// hoist every op's argument loads out of the loop (which would exhaust the
// scalar registers and spill).
using KArgs = const __attribute__((address_space(4))) Args;

__device__ __forceinline__ KArgs& kernel_args() {
  auto p = __builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return *(KArgs*)p;
}

// An instruction as the op bodies see it: the 32-byte record plus the step of
// a multi-step run it belongs to (0 outside mk_decode_loop).
struct Task : Instr {
  uint32_t step = 0;
};

// The 32-byte instruction record, read once and kept in scalar registers.
__device__ __forceinline__ Task load_instr(KArgs& a, uint32_t idx) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(a.instr + idx);
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k] = __builtin_amdgcn_readfirstlane(__builtin_nontemporal_load(p + k));
  Task in;
  in.op = (uint16_t)(w[0] & 0xFFFF); in.layer = (uint16_t)(w[0] >> 16);
  in.a0 = w[1]; in.a1 = w[2]; in.a2 = w[3]; in.wait_off = w[4]; in.wait_cnt = w[5]; in.signal = w[6]; in.n_wait = w[7];
  return in;
}

// ----------------------------------------------------------------------------- small helpers

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float -> bf16 bits, round to nearest, ties to even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {           // bf16 storage
  static constexpr int VEC = 1;               // 16-byte words per 8 elements
  __device__ static float get(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ static void put(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
  __device__ static float rounded(float v) { return bf16_to_f32(f32_to_bf16(v)); }
  __device__ static void unpack(const v4u* w, float f[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = __uint_as_float(w[0][k] << 16);
      f[2 * k + 1] = __uint_as_float(w[0][k] & 0xFFFF0000u);
    }
  }
};
template <> struct Elem<float> {
  static constexpr int VEC = 2;
  __device__ static float get(const float* p, size_t i) { return p[i]; }
  __device__ static void put(float* p, size_t i, float v) { p[i] = v; }
  __device__ static float rounded(float v) { return v; }
  __device__ static void unpack(const v4u* w, float f[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) { f[k] = __uint_as_float(w[0][k]); f[4 + k] = __uint_as_float(w[1][k]); }
  }
};

// Cross-lane helpers: DPP moves within a 16-lane row, lane permutes across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over the LPK (8 or 16) lanes of an aligned lane group; every lane gets it.
template <int LPK>
__device__ __forceinline__ float lane_group_sum(float v) {
  v += dpp_mov<0xB1>(v);                 // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);                 // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);                // row_half_mirror
  if constexpr (LPK == 16) v += dpp_mov<0x140>(v);   // row_mirror
  return v;
}
// Sum over the wave; every lane gets the same value.
__device__ __forceinline__ float wave_sum(float v) {
  v = lane_group_sum<16>(v);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}
// Exchange with the lane whose bit M differs (bits above M equal): lane
// permutes for bits 5 and 4, DPP mirrors and quad permutes within a row below.
template <int M>
__device__ __forceinline__ float xchg_bit(float v) {
  if constexpr (M == 5) return __shfl_xor(v, 32, 64);
  else if constexpr (M == 4) return __shfl_xor(v, 16, 64);
  else if constexpr (M == 3) return dpp_mov<0x140>(v);     // row_mirror: lane ^ 15 within the row
  else if constexpr (M == 2) return dpp_mov<0x141>(v);     // row_half_mirror: lane ^ 7 within 8
  else if constexpr (M == 1) return dpp_mov<0x4E>(v);      // quad_perm [2,3,0,1]
  else return dpp_mov<0xB1>(v);                            // quad_perm [1,0,3,2]
}
// Sums of N values per lane over the wave, N a power of two up to 64, with
// about two exchanges per value instead of one full reduction each: every
// step over lane bit M (5 down to 0) keeps half of the remaining values, the
// half chosen by that bit, and adds the partner's copy of it; once one value
// is left the steps just add.  On return v[0] of lane l is the total of value
// index l >> (6 - log2 N), identical in all lanes of that index.
template <int N, int M = 5>
__device__ __forceinline__ void wave_sum_many(float* v, int lane) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "power of two up to 64");
  if constexpr (M >= 0) {
    if constexpr (N > 1) {
      const bool hi = (lane >> M) & 1;
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        const float keep = hi ? v[N / 2 + i] : v[i];
        const float send = hi ? v[i] : v[N / 2 + i];
        v[i] = keep + xchg_bit<M>(send);
      }
      wave_sum_many<N / 2, M - 1>(v, lane);
    } else {
      v[0] += xchg_bit<M>(v[0]);
      wave_sum_many<1, M - 1>(v, lane);
    }
  }
}
template <int N> constexpr int log2_of() { return N <= 1 ? 0 : 1 + log2_of<N / 2>(); }
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ----------------------------------------------------------------------------- barriers

// Trace record of instruction idx: TRACE_WORDS x u64, (workgroup << 32 | XCD),
// pop, waits ended, phase A, phase B, end (device wall clock).  Phase A / B
// mark the op body's inner steps (inputs staged / main loop done).
constexpr int TRACE_WORDS = 8;
__device__ __forceinline__ void trace_mark(KArgs& a, uint32_t idx, int slot) {
  if (a.trace && threadIdx.x == 0) a.trace[TRACE_WORDS * (size_t)idx + slot] = wall_clock64();
}

__device__ __forceinline__ bool aborted(KArgs& a) {
  return __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

__device__ inline void record_error(KArgs& a, uint32_t code, uint32_t idx, uint32_t bar, uint32_t val, uint32_t tgt) {
  uint32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(a.err, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)) {
    a.err[1] = idx; a.err[2] = bar; a.err[3] = val; a.err[4] = tgt;
  }
}

// Tile hand-off.  Intermediate tiles are written and read with device-coherent
// (agent-scope relaxed atomic) stores and loads, which bypass the per-XCD L2
// copies instead of relying on whole-cache write-back / invalidate; weights and
// the KV cache history are read-only during a step and use ordinary streaming
// loads.  A producer waits until its coherent stores are acknowledged, then one
// thread bumps the tile's counter; a consumer polls the counters of the tiles
// it reads and only then issues its coherent loads.
__device__ __forceinline__ void st_cg(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_cg(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 ld_cg4(const float* p) {          // 16-byte aligned
  uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<float*>(p));
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float4(__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
                     __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32)));
}

__device__ __forceinline__ int ld_cg_i32(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_cg_i32(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block until every barrier in the instruction's wait list reaches its target.
// Threads poll disjoint subsets.  Returns false if the wait gave up (timeout or
// another worker aborted).
__device__ __forceinline__ bool poll_counter(KArgs& a, const uint32_t* ctr, uint32_t tgt, uint32_t idx, uint32_t id) {
  uint32_t spins = 0, v;
  while ((v = __hip_atomic_load(const_cast<uint32_t*>(ctr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < tgt) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins >= a.spin_limit) { record_error(a, ERR_TIMEOUT, idx, id, v, tgt); return false; }
    if ((spins & 255) == 0 && aborted(a)) return false;
  }
  return true;
}

// Counters are cleared once per launch: in step t of a multi-step run a barrier
// of the same step is complete at target * (t + 1) signals, one of the previous
// step (a wait range whose count has bit 31 set) at target * t.
__device__ __forceinline__ bool wait_tiles(KArgs& a, const Task in, uint32_t idx) {
  bool ok = true;
  for (uint32_t k = 0; k < in.wait_cnt; ++k) {
    const Range rg = a.ranges[in.wait_off + k];
    const uint32_t cnt = rg.count & 0x7FFFFFFFu;
    const uint32_t mul = (rg.count & 0x80000000u) ? in.step : in.step + 1;
    for (uint32_t j = threadIdx.x; j < cnt && ok; j += NT)
      ok = poll_counter(a, a.counters + rg.first + j, a.targets[rg.first + j] * mul, idx, rg.first + j);
  }
  const bool all = __syncthreads_and(ok) != 0;
  asm volatile("" ::: "memory");                 // no tile load may move above the wait
  trace_mark(a, idx, 2);
  return all;
}

// Race check (option MK_OPT_DELAY_SEED): before it stores its tile, a producer
// stalls for a pseudo-random time drawn from (seed, instruction index), 0 to
// about 50 us, so a consumer that read a tile without waiting for it would read
// the workspace's previous (poisoned) contents.  Uniform across the workgroup.
__device__ __forceinline__ void inject_delay(KArgs& a, uint32_t idx) {
  if (a.delay_seed == 0) return;
  uint32_t h = (idx + 1u) * 0x9E3779B1u ^ a.delay_seed;     // a 32-bit integer mix (murmur3 finaliser)
  h ^= h >> 16; h *= 0x85EBCA6Bu; h ^= h >> 13; h *= 0xC2B2AE35u; h ^= h >> 16;
  const uint32_t n = __builtin_amdgcn_readfirstlane(h & 15u);
  for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(127);
}

// Publish this instruction's tile: every wave waits for its coherent stores to
// be acknowledged, then one thread bumps the tile's counter.
__device__ __forceinline__ void signal_tile(KArgs& a, const Task in) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(a.counters + in.signal, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------------------- shared memory arena

// Views into the dynamic shared memory of a workgroup.  The host sizes the
// regions for the model and batch (Args::lds_*), so small models leave room
// for several workgroups per compute unit.  The GEMV staging buffer and the
// attention buffers share one region.
struct AttSmem {
  float* q;        // rotated queries            [r * hd]
  float* kn;       // new key, as stored          [hd]
  float* vn;       // new value, as stored        [hd]
  float* cs;       // rotary cos                  [hd / 2]
  float* sn;       // rotary sin                  [hd / 2]
  float* p;        // per-wave sums               [NWAVE * ATT_MAX_R]
  float* red;      // per-wave maxima             [NWAVE * ATT_MAX_R]
  float* part;     // per-wave outputs            [NWAVE * r * hd]
  float* stage_f;  // matrix-core GEMV input staging: the whole shared region
  int stage_floats;
};
struct Smem {
  uint32_t* idx;   // [0] current instruction index, [8..15] its record
  float* ss;       // per-row norm factors        [32]
  float* ssw;      // per-wave partial sums       [NWAVE * 32]
  float* res;      // GEMV results                [rows * NB]
  float* resid;    // residual rows of the tile   [rows * NB]
  uint8_t* ring;   // GEMV weight rings           [NWAVE][ring lines][1 KB]
  float* x;        // GEMV input staging          [xcap]
  int xcap;
  AttSmem att;
};

extern __shared__ __align__(16) float mk_smem[];

__device__ __forceinline__ Smem make_smem(KArgs& a) {
  Smem s;
  float* base = mk_smem;
  s.idx = reinterpret_cast<uint32_t*>(base);
  s.ss = base + 16;
  s.ssw = s.ss + 32;
  s.res = s.ssw + NWAVE * 32;
  s.resid = s.res + a.lds_res;
  float* u = s.resid + a.lds_res;
  s.ring = reinterpret_cast<uint8_t*>(u);
  s.x = u + a.lds_ring / 4;
  s.xcap = (int)a.lds_x;
  const int r = a.r, hd = a.hd;
  auto take = [&](int n) { float* p = u; u += (n + 3) & ~3; return p; };
  s.att.q = take(r * hd);
  s.att.kn = take(hd);
  s.att.vn = take(hd);
  s.att.cs = take(hd / 2);
  s.att.sn = take(hd / 2);
  s.att.p = take(NWAVE * ATT_MAX_R);
  s.att.red = take(NWAVE * ATT_MAX_R);
  s.att.part = take(NWAVE * r * hd);
  s.att.stage_f = reinterpret_cast<float*>(s.ring);       // weight ring, input staging and attention, as one region
  s.att.stage_floats = (int)a.lds_union;
  return s;
}

// ----------------------------------------------------------------------------- GEMV op bodies

// Weights stream through a per-wave ring of 1 KB lines in shared memory, filled
// by direct global->LDS loads (no registers held while in flight).  Lines are
// numbered in the order the wave consumes them; the ring is filled before the
// instruction waits on its producer tiles, then refilled one line per line
// consumed, so the ring's lines stay in flight per wave.

// One 16-byte-per-lane global->LDS load (64 lanes fill 1 KB at `lds`, lane i
// at lds + 16 i).  Issued through inline assembly so that the compiler does
// not treat every later shared-memory read as depending on it (it would wait
// for all outstanding loads before each read); the code that consumes the
// data waits for it explicitly with wait_vm.  POL 1 adds sc1 (device-coherent).
// The prefill GEMM pipeline and the decode GEMVs use it; the compiler's builtin
// remains as the MK_OPT_GEMV_PIPE = 2 variant of the decode GEMVs.
template <int POL>
__device__ __forceinline__ void dma_lds16(const void* src, void* lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)lds)));
  if constexpr (POL == 0)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(l) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off sc1" ::"v"(src), "s"(l) : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
}

// Rows come from up to two matrices: row i < split reads A[row0+i], row
// i >= split reads B[row0+i-split] (gate / up).  Each wave owns RPW rows of a
// pass of ROWS rows.
template <typename WT, int NB, int RPW, bool PIPE = false>
struct Gemv {
  static constexpr int ROWS = NWAVE * RPW;
  using E = Elem<WT>;
  static constexpr int LPI = E::VEC;     // lines per (row, 512-column iteration)

  const WT* A; const WT* B; int split; int row0; int nrows; int K;

  __device__ const WT* row_ptr(int i) const { return i < split ? A + (size_t)(row0 + i) * K : B + (size_t)(row0 + i - split) * K; }

  // Issue the RPW * LPI lines of one 512-column iteration `it` of pass `pass`
  // of this wave into ring group `grp`.  Lines of rows past the tile or
  // columns past K re-read valid addresses and are ignored by the consumer.
  __device__ void issue_iter(uint8_t* ring, int grp, int pass, int it, int wave, int lane) const {
    int col = it * 512 + lane * 8;
    if (col >= K) col = 0;
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      int row = pass * ROWS + wave * RPW + j;
      if (row >= nrows) row = 0;
      const WT* p = row_ptr(row) + col;
#pragma unroll
      for (int v = 0; v < LPI; ++v)
        if constexpr (PIPE) dma_lds16<0>(p + v * 4, ring + ((grp * RPW + j) * LPI + v) * 1024);
        else __builtin_amdgcn_global_load_lds(p + v * 4, ring + ((grp * RPW + j) * LPI + v) * 1024, 16, 0, 0);
    }
  }
};

// Stage x[b][k0:k0+kn] * gain into LDS; accumulate sum(x^2) per row when asked.
// The loads go out in batches of U per thread before any of them is used, so a
// chunk costs one memory round trip rather than one per element.  `resid`
// (nullable) adds s.resid[row * NB + b] = resid[b * resid_ld + row] for rows
// < resid_rows; the first NT of them are loaded in the same round trip.
template <int NB>
__device__ __forceinline__ void stage_x(Smem& s, const float* x, int ldx, int nb, int k0, int kn, const float* gain,
                                        bool want_ss, float ss[NB], const float* resid, int resid_ld, int resid_rows) {
  constexpr int U = 8;
  const int t = threadIdx.x;
  const bool has_r = resid && t < resid_rows * nb;
  const int rrow = has_r ? t / nb : 0, rb = has_r ? t - rrow * nb : 0;
  const float rv = has_r ? ld_cg(resid + (size_t)rb * resid_ld + rrow) : 0.f;
  const int q4 = kn >> 2;                                // float4 per row (kn is a multiple of 8)
  const int total = nb * q4;
  for (int u0 = t; u0 < total; u0 += NT * U) {
    float4 v[U], g[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = u0 + j * NT;
      if (u < total) {
        const int b = u / q4, k = (u - b * q4) * 4;
        v[j] = ld_cg4(x + (size_t)b * ldx + k0 + k);
        if (gain) g[j] = *reinterpret_cast<const float4*>(gain + k0 + k);
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = u0 + j * NT;
      if (u < total) {
        const int b = u / q4, k = (u - b * q4) * 4;
        float4 w = v[j];
        if (want_ss) {
          const float sq = w.x * w.x + w.y * w.y + w.z * w.z + w.w * w.w;
#pragma unroll
          for (int bb = 0; bb < NB; ++bb) if (bb == b) ss[bb] += sq;
        }
        if (gain) { w.x *= g[j].x; w.y *= g[j].y; w.z *= g[j].z; w.w *= g[j].w; }
        *reinterpret_cast<float4*>(s.x + b * kn + k) = w;
      }
    }
  }
  if (has_r) s.resid[rrow * NB + rb] = rv;
  // residual values beyond one per thread (many input rows)
  if (resid) {
    for (int e = t + NT; e < resid_rows * nb; e += NT) {
      const int row = e / nb, b = e - row * nb;
      s.resid[row * NB + b] = ld_cg(resid + (size_t)b * resid_ld + row);
    }
  }
}

// O-projection input rows of a queue whose split combines are fused into the
// O-projection: ATT[b][col] for all nb rows and the K = nq * hd columns, merged
// from the attention splits' partials (o | m | l per split, as COMBINE does)
// instead of read from ATT.  Every partial of the layer's nb rows is first
// copied into shared memory after the staged rows (one block of coherent
// 16-byte loads); the merge weights of each (row, KV head, query head) are
// computed once, then each column is one weighted sum over the splits.  The
// residual values are staged as stage_x does.  The host sizes the staging
// area for this.  Kept out of line: it is inlined into no GEMV body, so the
// unfused path's code stays as it was (the interpreter's size matters for the
// instruction cache).
template <int NB>
__device__ __attribute__((noinline)) void stage_att_fused(KArgs& a, Smem& s, int l, int nb, int K, const float* resid,
                                                int resid_ld, int resid_rows) {
  const int r = a.r, hd = a.hd, NS = a.NS, rhd = r * hd;
  const int slot_sz = rhd + 2 * r;
  float* P = s.x + NB * K;                                   // staged partials [nb][nkv][NS][slot]
  const float* src = a.OPART + l * a.sOP;
  const int total = nb * a.nkv * NS * slot_sz;
  const int t = threadIdx.x;
  const bool has_r = resid && t < resid_rows * nb;
  const int rrow = has_r ? t / nb : 0, rb = has_r ? t - rrow * nb : 0;
  const float rv = has_r ? ld_cg(resid + (size_t)rb * resid_ld + rrow) : 0.f;
  constexpr int U = 16;
  const int q4 = total >> 2;
  for (int u0 = t; u0 < q4; u0 += NT * U) {
    float4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) if (u0 + j * NT < q4) v[j] = ld_cg4(src + 4 * (u0 + j * NT));
#pragma unroll
    for (int j = 0; j < U; ++j) if (u0 + j * NT < q4) *reinterpret_cast<float4*>(P + 4 * (u0 + j * NT)) = v[j];
  }
  for (int e = 4 * q4 + t; e < total; e += NT) P[e] = ld_cg(src + e);
  if (has_r) s.resid[rrow * NB + rb] = rv;
  if (resid) {
    for (int e = t + NT; e < resid_rows * nb; e += NT) {
      const int row = e / nb, b = e - row * nb;
      s.resid[row * NB + b] = ld_cg(resid + (size_t)b * resid_ld + row);
    }
  }
  __syncthreads();
  // per (row, KV head, query head): split weights e^(m_s - m) / sum_s e^(m_s - m) l_s
  // (0 for empty splits), once, into shared memory after the partials
  float* W = P + total;                                      // [nb][nkv][r][NS]
  for (int e = t; e < nb * a.nkv * r; e += NT) {
    const int bg = e / r, h = e - bg * r;
    const float* pb = P + (size_t)bg * NS * slot_sz;
    float m = -INFINITY;
    for (int sp = 0; sp < NS; ++sp) m = fmaxf(m, pb[sp * slot_sz + rhd + h]);
    float den = 0.f;
    for (int sp = 0; sp < NS; ++sp) {
      const float ms = pb[sp * slot_sz + rhd + h];
      const float w = ms == -INFINITY ? 0.f : expf(ms - m);
      W[(size_t)e * NS + sp] = w;
      den = fmaf(w, pb[sp * slot_sz + rhd + r + h], den);
    }
    const float inv = 1.0f / den;
    for (int sp = 0; sp < NS; ++sp) W[(size_t)e * NS + sp] *= inv;
  }
  __syncthreads();
  for (int e = t; e < nb * K; e += NT) {
    const int b = e / K, col = e - b * K;
    const int g = col / rhd, o = col - g * rhd, h = o / hd;
    const float* pb = P + (size_t)(b * a.nkv + g) * NS * slot_sz + o;
    const float* w = W + ((size_t)(b * a.nkv + g) * r + h) * NS;
    float acc = 0.f;
    for (int sp = 0; sp < NS; ++sp) acc = fmaf(w[sp], pb[sp * slot_sz], acc);
    s.x[b * K + col] = acc;
  }
}

// Full GEMV of `nrows` rows against `nb` input rows of length K, results in
// s.res[row * NB + b] (already scaled by the row's RMSNorm factor when `norm`).
// The inputs are staged in column chunks as large as the shared memory allows;
// each chunk is staged once and every pass of RPW rows per wave runs over it
// before the next chunk, so the partial sums of a row add up in s.res across
// chunks (owned by one wave, in chunk order).  Each wave streams its rows'
// weight lines through its ring in that consumption order; the ring is filled
// before waiting on the instruction's producer tiles and refilled one group
// per group consumed.  `resid` (nullable) is staged with the first chunk:
// s.resid[row * NB + b] = resid[b * resid_ld + row].
// Returns false when the wait gave up.
template <typename WT, int NB, int RPW, bool PIPE>
__device__ __forceinline__ bool gemv(KArgs& a, Smem& s, const Gemv<WT, NB, RPW, PIPE>& g, const float* x, int nb,
                     const float* gain, bool norm, bool mega, bool fused, const Task in, uint32_t idx,
                     const float* resid, int resid_ld) {
  using G = Gemv<WT, NB, RPW, PIPE>;
  using E = Elem<WT>;
  const int K = g.K;
  const int iters = (K + 511) / 512;
  const int ipc = (s.xcap / NB) / 512;                 // 512-column iterations per staged chunk
  const int kc_max = ipc * 512;
  const int nch = (iters + ipc - 1) / ipc;
  const int npass = (g.nrows + G::ROWS - 1) / G::ROWS;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  constexpr int RING_LINES = ring_lines<NB>();
  uint8_t* ring = s.ring + wave * RING_LINES * 1024;
  constexpr int GL = RPW * G::LPI;                     // lines per iteration group
  constexpr int NG = RING_LINES / GL;                  // groups in the ring
  static_assert(NG >= 2, "ring holds at least two iteration groups");   // whole groups; spare lines unused
  const int ngroups = npass * iters;                   // groups this wave consumes
  // refill cursor: the next (chunk, pass, iteration) to issue
  int rb = 0, re = min(ipc, iters), rp = 0, ri = 0;   // chunk [rb, re) of iterations
  auto issue_next = [&](int grp) {
    g.issue_iter(ring, grp, rp, ri, wave, lane);
    if (++ri == re) {
      ri = rb;
      if (++rp == npass) { rp = 0; rb = re; re = min(re + ipc, iters); ri = rb; }
    }
  };
  for (int q = 0; q < min(ngroups, NG); ++q) issue_next(q);          // prefetch
  if (mega && !wait_tiles(a, in, idx)) {
    wait_vm<0>();                                        // drain before the ring is reused
    return false;
  }

  float ssl[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) ssl[b] = 0.f;
  int gi = 0;                                            // next group to consume

  for (int ci = 0; ci < nch; ++ci) {
    const int kc0 = ci * kc_max;
    const int kcn = min(kc_max, K - kc0);
    if (ci > 0) __syncthreads();                         // every wave is done with the previous chunk
    if (!fused) stage_x<NB>(s, x, K, nb, kc0, kcn, gain, norm, ssl, ci == 0 ? resid : nullptr, resid_ld, g.nrows);
    else stage_att_fused<NB>(a, s, in.layer, nb, K, resid, resid_ld, g.nrows);   // one chunk (host-sized)
    __syncthreads();
    if (mega && ci == 0) trace_mark(a, idx, 3);
    const int it_begin = kc0 / 512, it_end = (kc0 + kcn + 511) / 512;
    for (int pass = 0; pass < npass; ++pass) {
      float acc[RPW][NB];
#pragma unroll
      for (int j = 0; j < RPW; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[j][b] = 0.f;
      for (int it = it_begin; it < it_end; ++it, ++gi) {
        const int col = it * 512 + lane * 8;
        const bool valid = col < K;
        // batched inputs: columns past K read column 0 and their weights are zeroed below
        const int c = (NB <= 2 || valid) ? col - kc0 : 0;
        // group gi has landed once at most (issued - gi - 1) groups are outstanding
        if (gi + NG <= ngroups) wait_vm<(NG - 1) * GL>(); else wait_vm<0>();
        const uint8_t* gbase = ring + (gi % NG) * GL * 1024 + lane * 16;
        v4u w[RPW][G::LPI];
#pragma unroll
        for (int j = 0; j < RPW; ++j)
#pragma unroll
          for (int v = 0; v < G::LPI; ++v) w[j][v] = *reinterpret_cast<const v4u*>(gbase + (j * G::LPI + v) * 1024);
        // the group's reads have returned: its slots can be refilled
        __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0); vmcnt, expcnt unconstrained
        if (gi + NG < ngroups) issue_next(gi % NG);
        float wf[RPW][8];
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
          E::unpack(w[j], wf[j]);
          if (NB > 2 && (K & 511) && !valid) {
#pragma unroll
            for (int e = 0; e < 8; ++e) wf[j][e] = 0.f;
          }
        }
        // one input row at a time against all of the wave's rows.  Batched
        // inputs read without branches: rows past nb read whatever the staging
        // area holds (in bounds: NB * kc_max <= xcap) and their sums are never
        // stored.  One or two rows keep the branch (measured faster there).
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          float xv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          if (NB > 2 || (b < nb && valid)) {
            const float4 x0 = *reinterpret_cast<const float4*>(s.x + b * kcn + c);
            const float4 x1 = *reinterpret_cast<const float4*>(s.x + b * kcn + c + 4);
            xv[0] = x0.x; xv[1] = x0.y; xv[2] = x0.z; xv[3] = x0.w;
            xv[4] = x1.x; xv[5] = x1.y; xv[6] = x1.z; xv[7] = x1.w;
          }
#pragma unroll
          for (int j = 0; j < RPW; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[j][b] = fmaf(wf[j][e], xv[e], acc[j][b]);
        }
      }
      // reduce every (row, b) across the wave at once; the first lane holding
      // a total adds it to the row's sum
      constexpr int NV = RPW * NB, SH = 6 - log2_of<NV>();
      wave_sum_many<NV>(&acc[0][0], lane);
      {
        const int vi = lane >> SH, j = vi / NB, b = vi - j * NB;
        const int row = pass * G::ROWS + wave * RPW + j;
        if ((lane & ((1 << SH) - 1)) == 0 && row < g.nrows && b < nb)
          s.res[row * NB + b] = ci == 0 ? acc[0][0] : s.res[row * NB + b] + acc[0][0];
      }
    }
  }
  if (mega) trace_mark(a, idx, 4);
  if (norm) {
    // every thread staged a disjoint part of the rows: reduce sum(x^2) over the workgroup
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float v = wave_sum(ssl[b]);
      if (lane == 0) s.ssw[wave * 32 + b] = v;
    }
    __syncthreads();
    if (threadIdx.x < nb) {
      float t = 0.f;
      for (int w = 0; w < NWAVE; ++w) t += s.ssw[w * 32 + threadIdx.x];
      s.ss[threadIdx.x] = 1.0f / sqrtf(t / (float)K + a.eps);
    }
  }
  __syncthreads();
  if (norm) {
    for (int e = threadIdx.x; e < g.nrows * nb; e += NT) {
      const int row = e / nb, b = e - row * nb;
      s.res[row * NB + b] *= s.ss[b];
    }
    __syncthreads();
  }
  return true;
}

// Batched GEMV on the matrix cores (up to 32 input rows, bf16 weights, at most
// 128 weight rows, K a multiple of the step width CC below).  With several input rows the vector
// units' FMAs, not HBM, bound a GEMV; v_mfma_f32_32x32x16_bf16 takes the
// weight rows as A rows (RG groups of 32) and the input rows as B columns.
// Each product is taken twice, with y = x (.) gain split per element into bf16
// hi and lo parts (about 16 bits of y against the exact bf16 weights; fp32
// accumulation), as in the prefill GEMMs and the batched LM head.  Lane l
// holds A row / B column l % 32; within a 64-column block its K step q carries
// columns 32 (l / 32) + 8 q .. + 8 of both operands (one 64-byte piece of a
// weight row per lane and block).
//
// The work runs in steps of CC = 256 BPB columns, wave w taking BPB
// consecutive blocks of each.  A step's weights come straight into registers
// (one register set per step, the next step's set in flight while this one
// is multiplied, the first before the tile waits).  Its inputs are staged in
// shared memory (two buffers, rows padded by one float4 so that the lanes
// reading one column of 8 rows hit distinct banks): each thread loads
// its share of the next step's inputs (and of its gains) into registers before
// issuing the next weight set, and after this step's products the gains go to
// shared memory and the inputs, times their gains, to the other buffer.
// The waves add their sums into s.res in wave order.  Leaves what gemv leaves:
// s.res[row * NB + b] (normalised when asked) and s.resid.
// Columns per step of the matrix-core GEMV below (256 per block of each of the
// four waves: 4 / RG blocks, one at 3 or 4 row groups, at most 64 / NB so that
// a thread's share of a step's inputs stays at 16 float4s), and the floats of
// shared memory it stages (two input buffers and a step's gains) for a bucket
// of nb input rows.
constexpr int gemv_mfma_cc(int rg, int nb) {
  return 256 * ((rg >= 3 ? 1 : 4 / rg) < 64 / nb ? (rg >= 3 ? 1 : 4 / rg) : 64 / nb);
}
constexpr int gemv_mfma_floats(int cc, int nb) { return 2 * nb * (cc + 4) + cc; }
template <int RG, int NB>
struct MfmaGemvShape {
  static constexpr int CC = gemv_mfma_cc(RG, NB);       // columns per step
  static constexpr int BPB = CC / 256;                   // blocks per wave and step
  static constexpr int TPR = NT / NB;                    // staging threads per input row
  static constexpr int XF = CC / 4 / TPR;                // float4s per thread and step
};

template <int RGc, bool GAIN, typename WT, int NB, int RPW, bool PIPE>
__device__ __forceinline__ bool gemv_mfma_rg(KArgs& a, Smem& s, const Gemv<WT, NB, RPW, PIPE>& g, const float* x,
                                             int nb, const float* gain, bool norm, bool mega, const Task in,
                                             uint32_t idx, const float* resid, int resid_ld) {
  using SH = MfmaGemvShape<RGc, NB>;
  constexpr int BPB = SH::BPB, CC = SH::CC, TPR = SH::TPR, XF = SH::XF;
  static_assert(TPR >= 8 && TPR <= 64 && XF >= 1 && XF <= 16, "4 to 32 input rows");
  const int K = g.K, R = g.nrows;
  // the thread index, opaque to the optimiser: the lane offsets below are then
  // computed per call instead of being hoisted to the kernel's entry and
  // spilled (a reload from scratch inside the loop waits for every load in flight)
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int hf = lane >> 5, r = lane & 31;
  const int nstep = K / CC;                              // K is a multiple of CC (checked by the caller)
  constexpr int PS = CC + 4;                             // padded row stride (floats)
  float* xs = s.att.stage_f;                             // [2][NB][PS], then the step's gains [CC]
  float4* gs = reinterpret_cast<float4*>(xs + 2 * NB * PS);
  const WT* rp[RGc];
#pragma unroll
  for (int rg = 0; rg < RGc; ++rg) {
    const int row = rg * 32 + r;
    rp[rg] = g.row_ptr(row < R ? row : 0) + 32 * hf;
  }
  // Loads are unconditional, from pointers advanced in place by a uniform step
  // (no address temporaries, so the compiler counts every load in flight and
  // waits for exactly the set it multiplies); rows past R read row 0, unused,
  // and the set after the last is the last again.
  struct WB { v4u w[BPB * RGc][4]; };
  const v4u* wp[RGc];
#pragma unroll
  for (int rg = 0; rg < RGc; ++rg) wp[rg] = reinterpret_cast<const v4u*>(rp[rg] + 64 * wave * BPB);
  auto load_set = [&](WB& d, bool adv) {                 // the pointed-to set, then on to the next if adv
#pragma unroll
    for (int rg = 0; rg < RGc; ++rg) {
#pragma unroll
      for (int bi = 0; bi < BPB; ++bi)
#pragma unroll
        for (int q = 0; q < 4; ++q) d.w[bi * RGc + rg][q] = wp[rg][8 * bi + q];
      wp[rg] += adv ? 32 * BPB : 0;                      // 4 BPB blocks of 8 v4u
    }
  };
  df32x16 acc[RGc];
#pragma unroll
  for (int rg = 0; rg < RGc; ++rg)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[rg][v] = 0.f;
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  // the lane's first column of the wave's step, in B column r's staged row
  // (rows past nb hold row 0's inputs, unused)
  const float4* xl = reinterpret_cast<const float4*>(xs + r * PS) + 16 * wave * BPB + 8 * hf;
  auto mul_set = [&](const WB& d, int j) {
    const float4* xb = xl + (j & 1) * NB * (PS / 4);
#pragma unroll
    for (int bi = 0; bi < BPB; ++bi) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 x0 = xb[16 * bi + 2 * q];
        const float4 x1 = xb[16 * bi + 2 * q + 1];
        const float y[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        v4u hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){y[2 * e], y[2 * e + 1]}, bf2));
          hi[e] = h;
          lo[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
              (f2){y[2 * e] - __uint_as_float(h << 16), y[2 * e + 1] - __uint_as_float(h & 0xFFFF0000u)}, bf2));
        }
        const dbf16x8 bh = __builtin_bit_cast(dbf16x8, hi), bl = __builtin_bit_cast(dbf16x8, lo);
#pragma unroll
        for (int rg = 0; rg < RGc; ++rg) {
          const dbf16x8 af = __builtin_bit_cast(dbf16x8, d.w[bi * RGc + rg][q]);
          acc[rg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bh, acc[rg], 0, 0, 0);
          acc[rg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bl, acc[rg], 0, 0, 0);
        }
      }
    }
  };
  // staging: thread t keeps input row t / TPR throughout (its sum of squares is
  // one register) and the float4 slots t % TPR + TPR u of each step
  const int sb = t / TPR, sq = t % TPR;
  const float* xrow = x + (size_t)(sb < nb ? sb : 0) * K;
  float4 xv[XF], gv;
  float ssl = 0.f;
  const float* xp = xrow + 4 * sq;
  const float* gp = GAIN ? gain + 4 * (t % (CC / 4)) : nullptr;
  auto issue_x = [&](bool adv) {                         // coherent loads of a step's inputs, and its gains
#pragma unroll
    for (int u = 0; u < XF; ++u) xv[u] = ld_cg4(xp + 4 * TPR * u);
    xp += adv ? CC : 0;
    if constexpr (GAIN) {
      gv = *reinterpret_cast<const float4*>(gp);
      gp += adv ? CC : 0;
    }
  };
  // ... times the gains, into buffer j & 1; the sums of squares count only
  // steps that exist.  Branch-free, so that no load is sunk past the next
  // weight set (a load issued after it would wait for all of that set).
  auto put_x = [&](int j, bool real) {
    if constexpr (GAIN) {
      gs[t % (CC / 4)] = gv;
      __syncthreads();
    }
    float4* xw = reinterpret_cast<float4*>(xs + ((j & 1) * NB + sb) * PS) + sq;
    const float4* gr = gs + sq;
#pragma unroll
    for (int u = 0; u < XF; ++u) {
      float4 v = xv[u];
      if constexpr (GAIN) {
        const float sqs = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        ssl += real ? sqs : 0.f;
        const float4 gg = gr[TPR * u];
        v.x *= gg.x; v.y *= gg.y; v.z *= gg.z; v.w *= gg.w;
      }
      xw[TPR * u] = v;
    }
  };
  WB wa, wb;
  load_set(wa, nstep > 1);                               // weights before the wait
  if (mega && !wait_tiles(a, in, idx)) return false;
  issue_x(nstep > 1);
  // residual rows of the tile (O-projection, down), by all threads
  if (resid) {
    for (int e = t; e < R * nb; e += NT) {
      const int row = e / nb, b = e - row * nb;
      s.resid[row * NB + b] = ld_cg(resid + (size_t)b * resid_ld + row);
    }
  }
  put_x(0, true);
  __syncthreads();
  if (mega) trace_mark(a, idx, 3);
  // step j: next inputs and weights in flight, products of step j, inputs of
  // step j + 1 into the other buffer (unrolled by two, so each register set
  // keeps its registers)
  auto step = [&](WB& cur, WB& nxt, int j) {
    const bool adv = j + 2 < nstep;                      // (uniform) step j + 2 exists
    issue_x(adv);
    load_set(nxt, adv);
    mul_set(cur, j);
    put_x(j + 1, j + 1 < nstep);
    __syncthreads();
  };
  for (int j = 0; j < nstep; j += 2) {
    step(wa, wb, j);
    if (j + 1 < nstep) step(wb, wa, j + 1);
  }
  if (mega) trace_mark(a, idx, 4);
  // each wave's sums into its own slice of the (now free) staging region, then
  // s.res = ((w0 + w1) + w2) + w3, times the row's norm factor when asked
  float* part = xs;                                      // [NWAVE][R][nb]
#pragma unroll
  for (int rg = 0; rg < RGc; ++rg)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = rg * 32 + 8 * (v / 4) + 4 * hf + (v % 4);
      if (row < R && r < nb) part[(wave * R + row) * nb + r] = acc[rg][v];
    }
  if (GAIN && norm) {
#pragma unroll
    for (int off = TPR / 2; off >= 1; off >>= 1) ssl += __shfl_xor(ssl, off, 64);
    if (sq == 0 && sb < nb) s.ss[sb] = 1.0f / sqrtf(ssl / (float)K + a.eps);
  }
  __syncthreads();
  for (int e = t; e < R * nb; e += NT) {
    const int row = e / nb, b = e - row * nb;
    float v = part[e];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) v += part[w * R * nb + e];
    s.res[row * NB + b] = GAIN && norm ? v * s.ss[b] : v;
  }
  __syncthreads();
  return true;
}

// Whether the matrix-core GEMV takes a tile: K a multiple of its step width,
// and the shared region holding its staging.
template <int NB>
__device__ __forceinline__ bool gemv_mfma_fits(const Smem& s, int nrows, int K) {
  const int cc = gemv_mfma_cc((nrows + 31) / 32, NB);
  return K % cc == 0 && gemv_mfma_floats(cc, NB) <= s.att.stage_floats;
}

template <typename WT, int NB, int RPW, bool PIPE>
__device__ __forceinline__ bool gemv_mfma(KArgs& a, Smem& s, const Gemv<WT, NB, RPW, PIPE>& g, const float* x, int nb,
                                          const float* gain, bool norm, bool mega, const Task in, uint32_t idx,
                                          const float* resid, int resid_ld) {
  // (the RMSNorm'd GEMVs carry a gain, the others none)
#define MK_MFMA_RG(RG)                                                                             \
  return gain ? gemv_mfma_rg<RG, true>(a, s, g, x, nb, gain, norm, mega, in, idx, resid, resid_ld) \
              : gemv_mfma_rg<RG, false>(a, s, g, x, nb, gain, norm, mega, in, idx, resid, resid_ld)
  switch ((g.nrows + 31) / 32) {
    case 1: MK_MFMA_RG(1);
    case 2: MK_MFMA_RG(2);
    case 3: MK_MFMA_RG(3);
    default: MK_MFMA_RG(4);
  }
#undef MK_MFMA_RG
}

// Rows per wave per pass: 4 (16-row passes) up to 16 input rows, 2 for 32
// (register pressure).  Tiles of at most 8 rows always use 2, so no wave
// streams placeholder rows.
template <int NB> constexpr int rpw_for() { return NB >= 32 ? 2 : 4; }

// The weight rows a GEMV instruction streams (op, layer, columns [a0, a1)),
// or false for other ops.
template <typename WT, int NB, int RPW, bool PIPE>
__device__ __forceinline__ bool gemv_of(KArgs& a, const Task in, Gemv<WT, NB, RPW, PIPE>& g) {
  const int l = in.layer, n0 = in.a0, n = in.a1 - in.a0;
  switch (in.op) {
    case mk::OP_QKV: {
      const WT* W = static_cast<const WT*>(a.wqkv) + (size_t)l * a.NQKV * a.H;
      g = {W, W, n, n0, n, a.H};
      return true;
    }
    case mk::OP_OPROJ: {
      const WT* W = static_cast<const WT*>(a.wo) + (size_t)l * a.H * a.NA;
      g = {W, W, n, n0, n, a.NA};
      return true;
    }
    case mk::OP_GATEUP: {
      const WT* Wg = static_cast<const WT*>(a.wgate) + (size_t)l * a.F * a.H;
      const WT* Wu = static_cast<const WT*>(a.wup) + (size_t)l * a.F * a.H;
      g = {Wg, Wu, n, n0, 2 * n, a.H};                  // rows >= n read the up matrix
      return true;
    }
    case mk::OP_DOWN: {
      const WT* W = static_cast<const WT*>(a.wdown) + (size_t)l * a.H * a.F;
      g = {W, W, n, n0, n, a.F};
      return true;
    }
    case mk::OP_LMHEAD: {                               // loop queues: LM-head rows [a0, a1)
      const WT* W = static_cast<const WT*>(a.lm_head);
      g = {W, W, n, n0, n, a.H};
      return true;
    }
    default:
      return false;
  }
}

// The GEMV ops: QKV (RMSNorm(X_l) Wqkv^T), OPROJ (X_l + ATT_l Wo^T), GATEUP
// (silu(RMSNorm(H) Wg^T) * (RMSNorm(H) Wu^T)) and DOWN (HRES_l + ACT_l Wd^T),
// each over output columns [a0, a1).
template <typename WT, int NB, int RPW, bool PIPE>
__device__ __forceinline__ void op_gemv_rpw(KArgs& a, Smem& s, const Task in, uint32_t idx, bool mega, bool fused) {
  using G = Gemv<WT, NB, RPW, PIPE>;
  const int l = in.layer, n0 = in.a0, n = in.a1 - in.a0;
  G g{};
  gemv_of<WT, NB, RPW, PIPE>(a, in, g);
  const int op = in.op;
  const float* x;
  const float* gain = nullptr;
  const float* resid = nullptr;
  int ld = 0;
  if (op == mk::OP_QKV) {
    x = a.X + l * a.sX; gain = a.attn_norm + (size_t)l * a.H;
  } else if (op == mk::OP_OPROJ) {
    x = fused ? nullptr : a.ATT + l * a.sATT; resid = a.X + l * a.sX + n0; ld = a.H;
  } else if (op == mk::OP_GATEUP) {
    x = a.HRES + l * a.sHRES; gain = a.ffn_norm + (size_t)l * a.H;
  } else if (op == mk::OP_LMHEAD) {
    x = a.lm_x; gain = a.final_norm;
  } else {
    x = a.ACT + l * a.sACT; resid = a.HRES + l * a.sHRES + n0; ld = a.H;
  }
  bool ok;
  if constexpr (NB >= MK_GEMV_MFMA_MIN_NB && sizeof(WT) == 2) {
    // batched rows on the matrix cores where the tile and its staged inputs fit
    if (!fused && g.nrows <= 128 && gemv_mfma_fits<NB>(s, g.nrows, g.K))
      ok = gemv_mfma<WT, NB, RPW, PIPE>(a, s, g, x, a.M, gain, gain != nullptr, mega, in, idx, resid, ld);
    else
      ok = gemv<WT, NB, RPW, PIPE>(a, s, g, x, a.M, gain, gain != nullptr, mega, fused, in, idx, resid, ld);
  } else {
    ok = gemv<WT, NB, RPW, PIPE>(a, s, g, x, a.M, gain, gain != nullptr, mega, fused, in, idx, resid, ld);
  }
  if (!ok) return;
  inject_delay(a, idx);
  {
    for (int e = threadIdx.x; e < n * a.M; e += NT) {
      const int row = e / a.M, b = e - row * a.M;
      if (op == mk::OP_QKV) {
        st_cg(a.QKV + l * a.sQKV + (size_t)b * a.NQKV + n0 + row, s.res[row * NB + b]);
      } else if (op == mk::OP_GATEUP) {
        const float gt = s.res[row * NB + b], up = s.res[(n + row) * NB + b];
        st_cg(a.ACT + l * a.sACT + (size_t)b * a.F + n0 + row, gt / (1.0f + expf(-gt)) * up);
      } else if (op == mk::OP_LMHEAD) {
        if (a.logits) a.logits[((size_t)in.step * a.M + b) * a.V + n0 + row] = s.res[row * NB + b];
      } else {
        float* out = op == mk::OP_OPROJ ? a.HRES + l * a.sHRES : a.X + (l + 1) * a.sX;
        st_cg(out + (size_t)b * a.H + n0 + row, s.resid[row * NB + b] + s.res[row * NB + b]);
      }
    }
  }
  if (op == mk::OP_LMHEAD && threadIdx.x < a.M) {
    // the tile's (largest logit, lowest index among equals) of each row, for the argmax
    const int b = threadIdx.x;
    float best = s.res[b];
    int bi = 0;
    for (int row = 1; row < n; ++row) {
      const float v = s.res[row * NB + b];
      if (v > best) { best = v; bi = row; }
    }
    st_cg(a.lm_val + (size_t)b * a.lm_blocks + n0 / LM_ROWS, best);
    st_cg_i32(a.lm_idx + (size_t)b * a.lm_blocks + n0 / LM_ROWS, n0 + bi);
  }
  if (mega) signal_tile(a, in);
}

template <typename WT, int NB>
// `fused`: an O-projection of a queue with fused split combines (merges the
// split partials itself).  The per-op kernels decide it at compile time (a
// separate O-projection kernel for fused queues), so the other per-op GEMV
// kernels carry none of its code or registers.
__device__ __forceinline__ void op_gemv(KArgs& a, Smem& s, const Task in, uint32_t idx, bool mega, bool fused) {
  constexpr int RPW = rpw_for<NB>();
  const int rows = (in.op == mk::OP_GATEUP ? 2 : 1) * (int)(in.a1 - in.a0);
  // Weight lines are issued so that the compiler does not serialise the ring
  // (with its builtin it waits for every line in flight before each read of the
  // staged inputs).  The compiler-ordered issue stays selectable
  // (MK_OPT_GEMV_PIPE = 2): 1.107 against 1.035 ms per step for the 1B shape at
  // batch 1.
  const bool pipe = a.gemv_pipe != 2;
  if (pipe) {
    if constexpr (RPW != 2) {
      if (rows <= 2 * NWAVE) { op_gemv_rpw<WT, NB, 2, true>(a, s, in, idx, mega, fused); return; }
    }
    op_gemv_rpw<WT, NB, RPW, true>(a, s, in, idx, mega, fused);
    return;
  }
  if constexpr (RPW != 2) {
    if (rows <= 2 * NWAVE) { op_gemv_rpw<WT, NB, 2, false>(a, s, in, idx, mega, fused); return; }
  }
  op_gemv_rpw<WT, NB, RPW, false>(a, s, in, idx, mega, fused);
}

// EMBED(n0, n1): X_0[b, n0:n1] = E[token_b, n0:n1]
template <typename WT>
__device__ __forceinline__ void op_embed(KArgs& a, const Task in, uint32_t idx, bool mega) {
  const int n0 = in.a0, n = in.a1 - in.a0;
  const WT* E = static_cast<const WT*>(a.embed);
  // loop queues: wait for the previous step's argmax (its tokens, and the end of
  // every reader of this tile in that step); single-step queues wait on nothing
  if (mega && in.wait_cnt && !wait_tiles(a, in, idx)) return;
  inject_delay(a, idx);
  for (int e = threadIdx.x; e < n * a.M; e += NT) {
    const int b = e / n, c = e - b * n;
    // a multi-step run with feedback embeds the previous step's argmax (written
    // in this launch by another workgroup: a device-coherent load)
    const int tok = (a.feedback && in.step > 0) ? ld_cg_i32(a.next_all + (size_t)(in.step - 1) * a.M + b)
                                                : a.tokens[(size_t)in.step * a.M + b];
    if (tok < 0 || tok >= a.V) {                 // out-of-range id: report, emit zeros
      if (c == 0) record_error(a, ERR_TOKEN, 0xFFFFFFFFu, (uint32_t)b, (uint32_t)tok, (uint32_t)a.V);
      st_cg(a.X + (size_t)b * a.H + n0 + c, 0.f);
      continue;
    }
    st_cg(a.X + (size_t)b * a.H + n0 + c, Elem<WT>::get(E, (size_t)tok * a.H + n0 + c));
  }
  if (mega) signal_tile(a, in);
}

// ----------------------------------------------------------------------------- attention

// Combine the lanes that share (lane % LPK) across the 64 / LPK groups.
template <int LPK, bool MAX>
__device__ __forceinline__ float across_groups(float v) {
  if constexpr (LPK == 8) {
    const float w = dpp_mov<0x128>(v);   // row_ror:8 = lane ^ 8
    v = MAX ? fmaxf(v, w) : v + w;
  }
#pragma unroll
  for (int o = 16; o < 64; o <<= 1) {
    const float w = __shfl_xor(v, o, 64);
    v = MAX ? fmaxf(v, w) : v + w;
  }
  return v;
}

// ATTN(b, g, s): partial attention of the r query heads of KV group g of row b
// over keys [s*kb, min((s+1)*kb, pos+1)), pos = ctx_lens[b].  Applies QK-norm
// and RoPE to q and the new k, writes the new k / v into the cache (in the
// split that holds pos), and stores (o, m, l) for the combine.
// ATTN(b, g, s): partial attention of the r query heads of KV group g of row b
// over keys [s * kb, min((s + 1) * kb, P_b + 1)), as (unnormalised o, max m,
// sum l) per head.  Lane mapping: HD / 8 lanes share a key, each holding 8
// of its dims, so a wave covers 64 / (HD / 8) keys per round and the
// workgroup 4x that; the dot products reduce over the key's lanes with
// shuffles, the softmax state lives in registers per key lane group, and the
// groups and waves merge once at the end.  The cached rows of the first 8
// rounds are loaded before the tile waits.
template <int HD>
__device__ __forceinline__ void attn_arrive(KArgs& a, Smem& s, const Task in, uint32_t idx);

template <typename KT, int HD>
__device__ __forceinline__ void op_attn(KArgs& a, Smem& s, const Task in, uint32_t idx, bool mega) {
  using E = Elem<KT>;
  constexpr int HALF = HD / 2;
  constexpr int NROT = ((ATT_MAX_R + 1) * HALF + NT - 1) / NT;
  constexpr int LPK = HD / 8;                       // lanes per key
  constexpr int KPW = 64 / LPK;                     // keys per wave per round
  constexpr int KPR = KPW * NWAVE;                  // keys per round
  constexpr int RPC = 8;                            // rounds per chunk (held in registers)
  constexpr int WPE = E::VEC;                       // 16-byte words per 8 elements
  const int l = in.layer, b = in.a0, g = in.a1, sp = in.a2;
  const int r = a.r;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int kk = lane / LPK, ds = lane % LPK;       // key of the lane in a round, its 8-dim slice
  const int pos_in = a.ctx_lens[b] + (int)in.step;      // step t of a run sits t positions on
  // a position outside the cache is reported and the row treated as having no keys
  const bool bad_pos = pos_in < 0 || pos_in >= a.ctx_max;
  if (bad_pos && t == 0 && sp == 0) record_error(a, ERR_CONTEXT, idx, (uint32_t)b, (uint32_t)pos_in, (uint32_t)a.ctx_max);
  const int pos = bad_pos ? -1 : pos_in;
  const int j0 = sp * a.kb, j1 = min(j0 + a.kb, pos + 1);
  const size_t head_off = (((size_t)l * a.M + b) * a.nkv + g) * (size_t)a.ctx_max;   // rows of this (l, b, g)
  KT* Kc = static_cast<KT*>(a.kc) + head_off * HD;
  KT* Vc = static_cast<KT*>(a.vc) + head_off * HD;
  auto key_of = [&](int rd) { return j0 + rd * KPR + wave * KPW + kk; };

  // this lane's 8-dim slices of the cached keys / values of one chunk of rounds;
  // rows without a cached key read as zeros (weight 0, never NaN * 0)
  v4u kr[RPC][WPE], vr[RPC][WPE];
  auto load_rows = [&](v4u (&dst)[RPC][WPE], const KT* base, int c0) {
#pragma unroll
    for (int rd = 0; rd < RPC; ++rd) {
      const int j = key_of(c0 + rd);
      if (j < j1 && j < pos) {
        const v4u* p = reinterpret_cast<const v4u*>(base + (size_t)j * HD + ds * 8);
#pragma unroll
        for (int w = 0; w < WPE; ++w) dst[rd][w] = __builtin_nontemporal_load(p + w);
      } else {
#pragma unroll
        for (int w = 0; w < WPE; ++w) dst[rd][w] = v4u{0u, 0u, 0u, 0u};
      }
    }
  };
  load_rows(kr, Kc, 0);
  load_rows(vr, Vc, 0);
  if (mega && !wait_tiles(a, in, idx)) return;
  inject_delay(a, idx);

  float* slot = a.OPART + l * a.sOP + ((size_t)(b * a.nkv + g) * a.NS + sp) * (size_t)(r * HD + 2 * r);
  if (j0 >= j1) {                                         // empty split
    for (int e = t; e < r * HD; e += NT) st_cg(slot + e, 0.f);
    if (t < r) { st_cg(slot + r * HD + t, -INFINITY); st_cg(slot + r * HD + r + t, 0.f); }
    if (a.merge_last) attn_arrive<HD>(a, s, in, idx);
    else if (mega) signal_tile(a, in);
    return;
  }

  // q (r heads), k, v of this row and group, then QK-norm and RoPE
  const float* qkv = a.QKV + l * a.sQKV + (size_t)b * a.NQKV;
  {
    // all of this row's q, k and v loads in flight at once (r * HD <= 2 * NT)
    float qv[2], kv = 0.f, vv = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) qv[j] = t + j * NT < r * HD ? ld_cg(qkv + g * r * HD + t + j * NT) : 0.f;
    if (t < HD) {
      kv = ld_cg(qkv + a.nq * HD + g * HD + t);
      vv = ld_cg(qkv + (a.nq + a.nkv) * HD + g * HD + t);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) if (t + j * NT < r * HD) s.att.q[t + j * NT] = qv[j];
    if (t < HD) { s.att.kn[t] = kv; s.att.vn[t] = vv; }
  }
  if (t < HALF) {
    // angle p * theta^(-2i/hd) in float64, reduced to [-pi, pi] in float64
    // (2 pi split in two parts), then evaluated in fp32
    const double ang = (double)pos * a.rope_inv[t];
    const double k = rint(ang * 0.15915494309189535);
    const double red = fma(-k, 6.283185307179586, ang) - k * 2.4492935982947064e-16;
    float sv, cv;
    sincosf((float)red, &sv, &cv);
    s.att.cs[t] = cv;
    s.att.sn[t] = sv;
  }
  __syncthreads();
  if (a.qk_norm) {
    // per-head RMSNorm over HD: one wave per head (the r query heads, then k)
    const int wave = t >> 6, lane = t & 63;
    for (int h = wave; h <= r; h += NWAVE) {
      float* v = h < r ? s.att.q + h * HD : s.att.kn;
      const float* gn = (h < r ? a.q_norm : a.k_norm) + (size_t)l * HD;
      float ss = 0.f;
      for (int d = lane; d < HD; d += 64) ss += v[d] * v[d];
      ss = wave_sum(ss);
      const float sc = 1.0f / sqrtf(ss / (float)HD + a.eps);
      for (int d = lane; d < HD; d += 64) v[d] = v[d] * sc * gn[d];
    }
    __syncthreads();
  }
  {
    // rotate pairs (i, i + HD/2) of every query head and of the key
    float y0[NROT], y1[NROT];
#pragma unroll
    for (int k = 0; k < NROT; ++k) {
      const int e = t + k * NT;
      if (e < (r + 1) * HALF) {
        const int h = e / HALF, i = e - h * HALF;
        const float* v = h < r ? s.att.q + h * HD : s.att.kn;
        const float x0 = v[i], x1 = v[i + HALF];
        y0[k] = x0 * s.att.cs[i] - x1 * s.att.sn[i];
        y1[k] = x1 * s.att.cs[i] + x0 * s.att.sn[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NROT; ++k) {
      const int e = t + k * NT;
      if (e < (r + 1) * HALF) {
        const int h = e / HALF, i = e - h * HALF;
        float* v = h < r ? s.att.q + h * HD : s.att.kn;
        v[i] = y0[k];
        v[i + HALF] = y1[k];
      }
    }
    __syncthreads();
  }
  // the new key / value are used as they will be read back from the cache
  if (t < HD) {
    const float kq = s.att.kn[t], vq = s.att.vn[t];
    if (j0 <= pos && pos < j1) {
      E::put(Kc, (size_t)pos * HD + t, kq);
      E::put(Vc, (size_t)pos * HD + t, vq);
    }
    s.att.kn[t] = E::rounded(kq);
    s.att.vn[t] = E::rounded(vq);
  }
  __syncthreads();
  if (mega) trace_mark(a, idx, 3);

  // registers: the lane's query slices, the new key / value slices, softmax state
  float qv[ATT_MAX_R][8], knv[8], vnv[8];
#pragma unroll
  for (int h = 0; h < ATT_MAX_R; ++h) {
    const float4 q0 = h < r ? *reinterpret_cast<const float4*>(s.att.q + h * HD + ds * 8) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 q1 = h < r ? *reinterpret_cast<const float4*>(s.att.q + h * HD + ds * 8 + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    qv[h][0] = q0.x; qv[h][1] = q0.y; qv[h][2] = q0.z; qv[h][3] = q0.w;
    qv[h][4] = q1.x; qv[h][5] = q1.y; qv[h][6] = q1.z; qv[h][7] = q1.w;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) { knv[e] = s.att.kn[ds * 8 + e]; vnv[e] = s.att.vn[ds * 8 + e]; }
  // scores are kept in log2 units (scaled by log2(e) / sqrt(HD)), so every
  // exponential is one v_exp_f32; m is converted back to natural units at the end
  constexpr float LOG2E = 1.4426950408889634f;
  const float scale = LOG2E / sqrtf((float)HD);
  float m_run[ATT_MAX_R], l_run[ATT_MAX_R], o_run[ATT_MAX_R][8];
#pragma unroll
  for (int h = 0; h < ATT_MAX_R; ++h) {
    m_run[h] = -INFINITY; l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o_run[h][e] = 0.f;
  }
  const int nrounds = (j1 - j0 + KPR - 1) / KPR;
  // The next chunk's keys are requested once this chunk's scores are formed and
  // its values once they are summed, so each load overlaps the other half.
  for (int c0 = 0; c0 < nrounds; c0 += RPC) {
    const bool more = c0 + RPC < nrounds;
    float sc[RPC][ATT_MAX_R];
#pragma unroll
    for (int rd = 0; rd < RPC; ++rd) {
      const int j = key_of(c0 + rd);
      float kf[8];
      E::unpack(kr[rd], kf);
      if (j == pos) {
#pragma unroll
        for (int e = 0; e < 8; ++e) kf[e] = knv[e];
      }
#pragma unroll
      for (int h = 0; h < ATT_MAX_R; ++h) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) p = fmaf(qv[h][e], kf[e], p);
        p = lane_group_sum<LPK>(p);
        sc[rd][h] = (j < j1 && h < r) ? p * scale : -INFINITY;
      }
    }
    if (more) load_rows(kr, Kc, c0 + RPC);
#pragma unroll
    for (int h = 0; h < ATT_MAX_R; ++h) {
      float mc = sc[0][h];
#pragma unroll
      for (int rd = 1; rd < RPC; ++rd) mc = fmaxf(mc, sc[rd][h]);
      const float mnew = fmaxf(m_run[h], mc);
      const float al = m_run[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[h] - mnew);
      l_run[h] *= al;
#pragma unroll
      for (int e = 0; e < 8; ++e) o_run[h][e] *= al;
      m_run[h] = mnew;
    }
#pragma unroll
    for (int rd = 0; rd < RPC; ++rd) {
      const int j = key_of(c0 + rd);
      float vf[8];
      E::unpack(vr[rd], vf);
      if (j == pos) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = vnv[e];
      }
#pragma unroll
      for (int h = 0; h < ATT_MAX_R; ++h) {
        const float p = sc[rd][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[rd][h] - m_run[h]);
        l_run[h] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) o_run[h][e] = fmaf(p, vf[e], o_run[h][e]);
      }
    }
    if (more) load_rows(vr, Vc, c0 + RPC);
  }
  if (mega) trace_mark(a, idx, 4);

  // merge the key lane groups of the wave (lanes with the same slice ds)
#pragma unroll
  for (int h = 0; h < ATT_MAX_R; ++h) {
    const float M = across_groups<LPK, true>(m_run[h]);
    const float f = m_run[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[h] - M);
    const float L = across_groups<LPK, false>(l_run[h] * f);
#pragma unroll
    for (int e = 0; e < 8; ++e) o_run[h][e] = across_groups<LPK, false>(o_run[h][e] * f);
    m_run[h] = M; l_run[h] = L;
  }
  // then the waves, through shared memory
  float* wo = s.att.part;                                 // [NWAVE][r * HD]
  float* wm = s.att.red;                                  // [NWAVE][ATT_MAX_R]
  float* wl = s.att.p;                                    // [NWAVE][ATT_MAX_R]
  if (kk == 0) {
#pragma unroll
    for (int h = 0; h < ATT_MAX_R; ++h) {
      if (h >= r) break;
#pragma unroll
      for (int e = 0; e < 8; ++e) wo[wave * r * HD + h * HD + ds * 8 + e] = o_run[h][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < ATT_MAX_R; ++h) { wm[wave * ATT_MAX_R + h] = m_run[h]; wl[wave * ATT_MAX_R + h] = l_run[h]; }
  }
  __syncthreads();
  for (int o = t; o < r * HD; o += NT) {
    const int h = o / HD;
    float M = wm[h];
    for (int w = 1; w < NWAVE; ++w) M = fmaxf(M, wm[w * ATT_MAX_R + h]);
    float num = 0.f;
    for (int w = 0; w < NWAVE; ++w) {
      const float mw = wm[w * ATT_MAX_R + h];
      if (mw != -INFINITY) num = fmaf(__builtin_amdgcn_exp2f(mw - M), wo[w * r * HD + o], num);
    }
    st_cg(slot + o, num);
  }
  if (t < r) {
    float M = wm[t];
    for (int w = 1; w < NWAVE; ++w) M = fmaxf(M, wm[w * ATT_MAX_R + t]);
    float L = 0.f;
    for (int w = 0; w < NWAVE; ++w) {
      const float mw = wm[w * ATT_MAX_R + t];
      if (mw != -INFINITY) L = fmaf(__builtin_amdgcn_exp2f(mw - M), wl[w * ATT_MAX_R + t], L);
    }
    st_cg(slot + r * HD + t, M * 0.6931471805599453f);          // back to natural units
    st_cg(slot + r * HD + r + t, L);
  }
  if (a.merge_last) attn_arrive<HD>(a, s, in, idx);
  else if (mega) signal_tile(a, in);
}

// Log-sum-exp merge of NS split partials (o[r*HD], m[r], l[r] per split, slot_sz
// floats apart, read through rd) into out[r*HD].
template <int HD, typename RD>
__device__ __forceinline__ void combine_rows(const float* src, float* out, int r, int NS, int slot_sz, RD rd) {
  constexpr int G8 = 8;
  auto part = [&](int e) { return rd(src + e); };
  for (int o = threadIdx.x; o < r * HD; o += NT) {
    const int h = o / HD;
    const int em = r * HD + h, el = r * HD + r + h;
    float m = -INFINITY;
    for (int sp0 = 0; sp0 < NS; sp0 += G8) {
      float v[G8];
#pragma unroll
      for (int j = 0; j < G8; ++j) v[j] = part(min(sp0 + j, NS - 1) * slot_sz + em);
#pragma unroll
      for (int j = 0; j < G8; ++j) m = fmaxf(m, v[j]);       // clamped repeats do not change the max
    }
    float num = 0.f, den = 0.f;
    for (int sp0 = 0; sp0 < NS; sp0 += G8) {
      float ms[G8], ov[G8], lv[G8];
#pragma unroll
      for (int j = 0; j < G8; ++j) {
        const int e = min(sp0 + j, NS - 1) * slot_sz;
        ms[j] = part(e + em); ov[j] = part(e + o); lv[j] = part(e + el);
      }
#pragma unroll
      for (int j = 0; j < G8; ++j) {
        if (sp0 + j >= NS || ms[j] == -INFINITY) continue;
        const float w = expf(ms[j] - m);
        num = fmaf(w, ov[j], num);
        den = fmaf(w, lv[j], den);
      }
    }
    st_cg(out + o, num / den);
  }
}

// Merge the NS split partials of row b, KV head g of layer l into ATT_l (the
// body of a COMBINE tile, or of the split that arrives last at (b, g)).
template <int HD>
__device__ __forceinline__ void merge_splits(KArgs& a, Smem& s, int l, int b, int g, bool mark, uint32_t idx) {
  const int r = a.r;
  const int slot_sz = r * HD + 2 * r;
  const int total = a.NS * slot_sz;
  const float* base = a.OPART + l * a.sOP + (size_t)(b * a.nkv + g) * a.NS * slot_sz;
  float* out = a.ATT + l * a.sATT + (size_t)b * a.NA + (size_t)g * r * HD;
  // all split partials at once into shared memory (independent coherent loads)
  const bool staged = total <= s.xcap;
  if (staged) {
    // 16-byte loads where the slots allow them: up to 12 K floats of partials
    // take a single round trip per thread
    const bool vec = (reinterpret_cast<uintptr_t>(base) & 15) == 0;
    const int q4 = vec ? total >> 2 : 0;
    constexpr int U4 = 12;
    for (int u0 = threadIdx.x; u0 < q4; u0 += NT * U4) {
      float4 v[U4];
#pragma unroll
      for (int j = 0; j < U4; ++j) if (u0 + j * NT < q4) v[j] = ld_cg4(base + 4 * (u0 + j * NT));
#pragma unroll
      for (int j = 0; j < U4; ++j)
        if (u0 + j * NT < q4) *reinterpret_cast<float4*>(s.x + 4 * (u0 + j * NT)) = v[j];
    }
    constexpr int U = 8;                                  // the rest: U scalar loads in flight at once
    for (int e0 = 4 * q4 + threadIdx.x; e0 < total; e0 += NT * U) {
      float v[U];
#pragma unroll
      for (int j = 0; j < U; ++j) if (e0 + j * NT < total) v[j] = ld_cg(base + e0 + j * NT);
#pragma unroll
      for (int j = 0; j < U; ++j) if (e0 + j * NT < total) s.x[e0 + j * NT] = v[j];
    }
    __syncthreads();
  }
  if (mark) trace_mark(a, idx, 3);
  // Splits are read eight at a time with clamped indices, so the loads of a
  // group are independent of each other and of the running max / sums (one
  // shared-memory round trip per eight splits rather than per split).
  if (staged) combine_rows<HD>(s.x, out, r, a.NS, slot_sz, [](const float* p) { return *p; });
  else combine_rows<HD>(base, out, r, a.NS, slot_sz, [](const float* p) { return ld_cg(p); });
}

// COMBINE(b, g): merge the NS split partials of row b, group g into ATT_l.
template <int HD>
__device__ __forceinline__ void op_combine(KArgs& a, Smem& s, const Task in, uint32_t idx, bool mega) {
  if (mega && !wait_tiles(a, in, idx)) return;
  inject_delay(a, idx);
  merge_splits<HD>(a, s, in.layer, in.a0, in.a1, mega, idx);
  if (mega) signal_tile(a, in);
}

// End of an attention split of a queue whose last split merges: count the
// arrival on the (row, KV head) partial tile, whose target is NS + 1.  The
// split whose count completes the NS arrivals (the fetch-add returns
// target * (step + 1) - 2) merges the partials: every other split stored its
// partial and waited for the stores' acknowledgement before its own count, so
// the partials are in place, as for a consumer whose poll has returned.  It
// then signals the tile once more, which is what the O-projection tiles wait
// for.  Runs in every execution mode (the per-op kernels clear the counters
// too).
template <int HD>
__device__ __forceinline__ void attn_arrive(KArgs& a, Smem& s, const Task in, uint32_t idx) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t before_last = a.targets[in.signal] * (in.step + 1) - 2;
    const uint32_t old =
        __hip_atomic_fetch_add(a.counters + in.signal, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s.idx[1] = old == before_last ? 1u : 0u;
  }
  __syncthreads();
  const uint32_t last = __builtin_amdgcn_readfirstlane(s.idx[1]);
  __syncthreads();
  if (!last) return;
  trace_mark(a, idx, 6);
  inject_delay(a, idx + a.n_instr);
  merge_splits<HD>(a, s, in.layer, in.a0, in.a1, false, idx);
  signal_tile(a, in);
}


// ARGMAX(b) (loop queues): the largest logit of row b over the LM-head tiles'
// partial maxima (lowest index among equals), stored as the step's next token.
__device__ __forceinline__ void op_argmax(KArgs& a, Smem& s, const Task in, uint32_t idx, bool mega) {
  if (mega && !wait_tiles(a, in, idx)) return;
  const int b = in.a0, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int k = t; k < a.lm_blocks; k += NT) {
    const float v = ld_cg(a.lm_val + (size_t)b * a.lm_blocks + k);
    const int i = ld_cg_i32(a.lm_idx + (size_t)b * a.lm_blocks + k);
    if (v > best || (v == best && i < bi)) { best = v; bi = i; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
  }
  if (lane == 0) { s.ssw[wave] = best; s.ssw[NWAVE + wave] = __int_as_float(bi); }
  __syncthreads();
  inject_delay(a, idx);
  if (t == 0) {
    for (int w = 1; w < NWAVE; ++w) {
      const float v = s.ssw[w];
      const int i = __float_as_int(s.ssw[NWAVE + w]);
      if (v > best || (v == best && i < bi)) { best = v; bi = i; }
    }
    st_cg_i32(a.next_all + (size_t)in.step * a.M + b, bi);
  }
  if (mega) signal_tile(a, in);
}

// ----------------------------------------------------------------------------- dispatch

// Per-op launch code of the O-projection of a queue with fused split combines
// (never an opcode of the queue: the records say OP_OPROJ).
constexpr int KPO_OPROJ_FUSED = 100;

template <typename WT, int NB, bool LOOP = false>
__device__ __forceinline__ void run_instr(KArgs& a, Smem& s, const Task in, uint32_t idx, bool mega, int only_op) {
  const int op = only_op ? only_op : in.op;
  switch (op) {
    case mk::OP_LMHEAD:                                  // loop queues only
      if constexpr (LOOP) op_gemv<WT, NB>(a, s, in, idx, mega, false);
      break;
    case mk::OP_ARGMAX:
      if constexpr (LOOP) op_argmax(a, s, in, idx, mega);
      break;
    case mk::OP_EMBED: op_embed<WT>(a, in, idx, mega); break;
    case mk::OP_QKV: case mk::OP_OPROJ: case mk::OP_GATEUP: case mk::OP_DOWN:
      // one GEMV body for the four ops (the interpreter's code size matters for
      // the instruction cache); only the megakernel's O-projection of a fused
      // queue merges split partials, a per-op kernel never does here
      op_gemv<WT, NB>(a, s, in, idx, mega, op == mk::OP_OPROJ && mega && a.fuse_combine);
      break;
    case KPO_OPROJ_FUSED:                                // per-op kernels only (folds away elsewhere)
      if (only_op == KPO_OPROJ_FUSED) op_gemv<WT, NB>(a, s, in, idx, mega, true);
      break;
    case mk::OP_ATTN:
      if (a.hd == 64) op_attn<WT, 64>(a, s, in, idx, mega); else op_attn<WT, 128>(a, s, in, idx, mega);
      break;
    case mk::OP_COMBINE:
      if (a.hd == 64) op_combine<64>(a, s, in, idx, mega); else op_combine<128>(a, s, in, idx, mega);
      break;
    default:
      if (threadIdx.x == 0) record_error(a, ERR_OPCODE, idx, in.op, 0, 0);
      break;
  }
}

// The persistent interpreter: pop, decode, run (wait -> compute -> signal).
// The pop of the next instruction is issued before the current one runs, so
// its round trip overlaps the current instruction's loads; with one sub-queue
// per worker there is nothing to pop.  Sub-queue q holds
// instructions q, q + n_queues, ... in queue order; every sub-queue is a
// subsequence of one topological order, so popping ahead cannot deadlock.
// LOOP (persistent multi-step decode, loop queues): the sequence is the queue
// repeated a.steps times, position k being instruction k mod n_instr of step
// k / n_instr; the repeated queue is still in topological order (a step's
// embedding waits only on the previous step's argmax), so the same argument
// holds and the host launches once for all steps.
template <typename WT, int NB, bool LOOP = false, bool POP = false>
__global__ __launch_bounds__(NT) void mk_interp(Args args) {
  Smem s = make_smem(kernel_args());
  const uint32_t nq = args.n_queues;
  const uint32_t qi = blockIdx.x % nq;
  const uint64_t total = LOOP ? (uint64_t)args.n_instr * (uint64_t)args.steps : args.range_end;
  // One sub-queue per worker: the worker runs positions qi, qi + nq, ... and
  // needs no pops; each instruction's record is loaded one iteration ahead.
  const bool fixed = nq == gridDim.x;
  auto instr_of = [&](uint64_t k) -> uint32_t {
    if constexpr (LOOP) return (uint32_t)(k % args.n_instr);
    else return (uint32_t)k;
  };
  uint32_t k_next = 0;                           // thread 0 (shared sub-queues): popped position
  uint32_t abort_seen = 0;                       // thread 0: error word, read one instruction ago
  uint32_t word = 0;                             // lanes 0..7 (fixed): next record, in flight
  if (threadIdx.x == 0 && !fixed) {
    KArgs& a = kernel_args();
    k_next = __hip_atomic_fetch_add(a.heads + qi * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // a launch of a composition starts at its range's first position of this worker
  const uint32_t it0 = (!LOOP && fixed && args.range_begin > qi) ? (args.range_begin - qi + nq - 1) / nq : 0;
  if (fixed && threadIdx.x < 8 && (uint64_t)qi + (uint64_t)it0 * nq < total) {
    KArgs& a = kernel_args();
    word = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a.instr + instr_of(qi + it0 * nq)) +
                                      threadIdx.x);
  }
  for (uint32_t it = it0;; ++it) {
    KArgs& a = kernel_args();
    const uint64_t fi = (uint64_t)qi + (uint64_t)it * nq;         // fixed order: this iteration's position
    if (threadIdx.x == 0) {
      const uint64_t k = fixed ? fi : (uint64_t)k_next * nq + qi;
      const bool go = k < total && abort_seen == 0;
      s.idx[0] = go ? (uint32_t)k : 0xFFFFFFFFu;
      if (go && !fixed)
        k_next = __hip_atomic_fetch_add(a.heads + qi * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // a worker that recorded an error stops the others at their next pop; the
      // read's round trip overlaps this instruction
      abort_seen = __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (fixed && threadIdx.x < 8) {
      s.idx[8 + threadIdx.x] = word;             // this instruction's record, loaded an iteration ago
      const uint64_t j = fi + nq;
      word = j < total ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a.instr + instr_of(j)) + threadIdx.x)
                       : 0u;
    }
    __syncthreads();
    const uint32_t pos = __builtin_amdgcn_readfirstlane(s.idx[0]);   // uniform: keep the record in SGPRs
    Task in;
    if (fixed) {
      uint32_t w[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) w[k] = __builtin_amdgcn_readfirstlane(s.idx[8 + k]);
      in.op = (uint16_t)(w[0] & 0xFFFF); in.layer = (uint16_t)(w[0] >> 16);
      in.a0 = w[1]; in.a1 = w[2]; in.a2 = w[3]; in.wait_off = w[4]; in.wait_cnt = w[5]; in.signal = w[6]; in.n_wait = w[7];
    }
    __syncthreads();
    if (pos == 0xFFFFFFFFu) break;
    const uint32_t idx = instr_of(pos);
    if (!fixed) in = load_instr(a, idx);
    if constexpr (LOOP) in.step = pos / a.n_instr;
    if constexpr (!POP) {
      unsigned long long t0 = 0;
      if (a.trace) t0 = wall_clock64();
      run_instr<WT, NB, LOOP>(a, s, in, idx, true, 0);
      if (a.trace && threadIdx.x == 0) {
        unsigned long long* rec = a.trace + TRACE_WORDS * (size_t)idx;
        uint32_t xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        rec[0] = ((unsigned long long)blockIdx.x << 32) | (xcc & 0xF);
        rec[1] = t0;
        rec[5] = wall_clock64();
      }
      continue;
    }
    // Run-time hand-out of a layer's splits (the POP variant: plan attn_pop,
    // one sub-queue per worker): at its first split position of a layer the
    // worker takes splits in queue order from the layer's counter until none
    // are left (each still waits on and signals its own tiles), then skips its
    // other positions in the layer's split segment, which the counter has
    // handed out.  One call site of the op bodies serves both orders.
    const bool pop = fixed && in.op == mk::OP_ATTN;
    const uint32_t f0 = pop ? a.attn_first + in.layer * a.attn_stride : 0, cnt = a.attn_count;
    Task cur = in;
    uint32_t id = idx;
    for (;;) {
      if (pop) {
        if (threadIdx.x == 0) {                  // (a recorded error ends the hand-out)
          const uint32_t t = __hip_atomic_fetch_add(a.heads + (a.n_queues + in.layer) * 32, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
          s.idx[2] = aborted(a) ? cnt : t;
        }
        __syncthreads();
        const uint32_t tk = __builtin_amdgcn_readfirstlane(s.idx[2]);
        __syncthreads();
        if (tk >= cnt) break;
        id = f0 + tk;
        cur = load_instr(a, id);
      }
      unsigned long long t0 = 0;
      if (a.trace) t0 = wall_clock64();
      run_instr<WT, NB, LOOP>(a, s, cur, id, true, 0);
      if (a.trace && threadIdx.x == 0) {
        unsigned long long* rec = a.trace + TRACE_WORDS * (size_t)id;
        uint32_t xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        rec[0] = ((unsigned long long)blockIdx.x << 32) | (xcc & 0xF);
        rec[1] = t0;
        rec[5] = wall_clock64();
      }
      if (!pop) break;
    }
    if (pop) {
      // the first iteration whose position lies past the segment runs next
      it = (f0 + cnt - qi + nq - 1) / nq - 1;
      if (threadIdx.x < 8) {
        const uint64_t j = (uint64_t)qi + (uint64_t)(it + 1) * nq;
        word = j < total ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a.instr + instr_of(j)) + threadIdx.x)
                         : 0u;
      }
    }
  }
  wait_vm<0>();                                  // no weight loads may outlive the workgroup
}

// Multi-stream mode (MegaOps abstract: dependent kernels overlap and
// synchronise on tiles of the intermediate tensor instead of at kernel
// boundaries): one launch per (layer, op) segment, on one of several streams;
// its workgroups stride over the segment's instructions and every instruction
// waits on and signals the same tile counters as in the megakernel.  The host
// caps each launch's workgroups so that the kernels that can be running at
// once (one per stream) are all resident together.
template <typename WT, int NB, int OP>
__global__ __launch_bounds__(NT) void ms_kernel(Args args, uint32_t first, uint32_t count) {
  KArgs& a = kernel_args();
  Smem s = make_smem(a);
  for (uint32_t i = blockIdx.x; i < count; i += gridDim.x) {
    // an error recorded anywhere (a wait that gave up) stops the remaining
    // instructions instead of letting each of them wait out its own limit
    if (threadIdx.x == 0) s.idx[0] = __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t abort_seen = __builtin_amdgcn_readfirstlane(s.idx[0]);
    __syncthreads();
    if (abort_seen) break;
    const uint32_t idx = first + i;
    const Task in = load_instr(a, idx);
    if (in.op != (OP == KPO_OPROJ_FUSED ? mk::OP_OPROJ : OP)) {
      if (threadIdx.x == 0) record_error(a, ERR_OPCODE, idx, in.op, 0, 0);
      break;                                               // uniform: every thread read the same record
    }
    // the GEMV ops are specialised at compile time (the O-projection of a queue
    // without fused combines need not carry the merge's registers)
    if constexpr (OP == mk::OP_QKV || OP == mk::OP_OPROJ || OP == mk::OP_GATEUP || OP == mk::OP_DOWN)
      op_gemv<WT, NB>(a, s, in, idx, true, false);
    else if constexpr (OP == KPO_OPROJ_FUSED)
      op_gemv<WT, NB>(a, s, in, idx, true, true);
    else
      run_instr<WT, NB>(a, s, in, idx, true, OP);
  }
  wait_vm<0>();                                            // no weight loads may outlive the workgroup
}

// One launch per (layer, op): workgroup i runs instruction first + i, no waits.
template <typename WT, int NB, int OP>
__global__ __launch_bounds__(NT) void kpo_kernel(Args args, uint32_t first) {
  KArgs& a = kernel_args();
  Smem s = make_smem(a);
  const uint32_t idx = first + blockIdx.x;
  const Task in = load_instr(a, idx);
  if (in.op != (OP == KPO_OPROJ_FUSED ? mk::OP_OPROJ : OP)) {
    if (threadIdx.x == 0) record_error(a, ERR_OPCODE, idx, in.op, 0, 0);
    return;
  }
  run_instr<WT, NB>(a, s, in, idx, false, OP);
}

// LM head on the matrix cores for 2 to 32 rows of bf16 weights (where the
// register-streaming kernel does not take them): at several rows the head is a
// skinny GEMM [M x H] x [H x V], which the vector units run at a fraction of
// the HBM rate.  logits[b][v] = rms_b^-1 * sum_k y_b[k]
// W[v][k] with y_b = x_b (.) g.  A first kernel writes y split per element into
// bf16 hi and lo parts (each product is taken twice, as in the prefill GEMMs:
// about 16 bits of y against the exact bf16 weights) and rms_b^-1; the
// products accumulate in fp32.
//
// lm_prep_kernel: one workgroup per row.
template <typename WT>
__global__ __launch_bounds__(NT) void lm_prep_kernel(Args args) {
  KArgs& a = kernel_args();
  __shared__ float red[NWAVE];
  const int b = blockIdx.x, H = a.H;
  const float* x = a.lm_x + (size_t)b * H;
  uint16_t* yh = a.lm_y + (size_t)b * H;
  uint16_t* yl = a.lm_y + ((size_t)a.M + b) * H;
  float ss = 0.f;
  for (int k = 8 * threadIdx.x; k < H; k += 8 * NT) {
    const float4 x0 = *reinterpret_cast<const float4*>(x + k), x1 = *reinterpret_cast<const float4*>(x + k + 4);
    const float4 g0 = *reinterpret_cast<const float4*>(a.final_norm + k);
    const float4 g1 = *reinterpret_cast<const float4*>(a.final_norm + k + 4);
    const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    v4u hi, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ss = fmaf(xv[2 * e], xv[2 * e], ss);
      ss = fmaf(xv[2 * e + 1], xv[2 * e + 1], ss);
      const float y0 = xv[2 * e] * gv[2 * e], y1 = xv[2 * e + 1] * gv[2 * e + 1];
      const uint32_t h0 = f32_to_bf16(y0), h1 = f32_to_bf16(y1);
      hi[e] = h0 | (h1 << 16);
      lo[e] = (uint32_t)f32_to_bf16(y0 - bf16_to_f32(h0)) | ((uint32_t)f32_to_bf16(y1 - bf16_to_f32(h1)) << 16);
    }
    *reinterpret_cast<v4u*>(yh + k) = hi;
    *reinterpret_cast<v4u*>(yl + k) = lo;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.f;
    for (int w = 0; w < NWAVE; ++w) tot += red[w];
    a.lm_rs[b] = 1.0f / sqrtf(tot / (float)H + a.eps);
  }
}

// lm_head_mfma: v_mfma_f32_32x32x16_bf16 with the vocabulary as the A rows and
// the batch rows (zero past M) as the B columns.  Lane l holds A row / B
// column l % 32; within a 64-column block its K step s carries columns
// 32 (l / 32) + 8 s .. + 8 of both operands (one 64-byte piece of a weight row
// per lane and block, the same permutation of k on both sides).  Wave w of
// workgroup i owns vocabulary rows 512 i + 128 w .. + 128 as four 32-row
// tiles; a block's weights and rows are loaded one block ahead.  Also writes
// each 64-row block's (max, lowest index) per row for the argmax.
constexpr int LMM_ROWS = 512;              // vocabulary rows per workgroup
template <typename WT>                     // bf16 weights (uint16_t) only
__global__ __launch_bounds__(NT) void lm_head_mfma(Args args) {
  static_assert(sizeof(WT) == 2, "bf16 weights");
  KArgs& a = kernel_args();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hf = lane >> 5, j = lane & 31;
  const int H = a.H, V = a.V, M = a.M;
  const int v0 = blockIdx.x * LMM_ROWS + wave * 128;
  const WT* W = static_cast<const WT*>(a.lm_head);
  const bool row_ok = j < M;
  const uint16_t* yh = a.lm_y + (size_t)(row_ok ? j : 0) * H + 32 * hf;
  const uint16_t* yl = a.lm_y + ((size_t)M + (row_ok ? j : 0)) * H + 32 * hf;
  // the lane's four weight rows (clamped inside the vocabulary; rows past it are never stored)
  const WT* wr[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) wr[t] = W + (size_t)min(v0 + 32 * t + j, V - 1) * H + 32 * hf;
  struct Blk { v4u w[4][4]; v4u h[4], l[4]; };
  auto load = [&](Blk& bk, int kb) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const v4u* p = reinterpret_cast<const v4u*>(wr[t] + kb);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) bk.w[t][s4] = p[s4];      // cached: the four pieces share a line
    }
    const v4u* ph = reinterpret_cast<const v4u*>(yh + kb);
    const v4u* pl = reinterpret_cast<const v4u*>(yl + kb);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      bk.h[s4] = row_ok ? ph[s4] : v4u{0u, 0u, 0u, 0u};
      bk.l[s4] = row_ok ? pl[s4] : v4u{0u, 0u, 0u, 0u};
    }
  };
  df32x16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.f;
  auto mul = [&](const Blk& bk) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const dbf16x8 bh = __builtin_bit_cast(dbf16x8, bk.h[s4]), bl = __builtin_bit_cast(dbf16x8, bk.l[s4]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const dbf16x8 af = __builtin_bit_cast(dbf16x8, bk.w[t][s4]);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bh, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bl, acc[t], 0, 0, 0);
      }
    }
  };
  // blocks of 64 columns in pairs: the next block's loads go out before a block is multiplied
  Blk ba, bb;
  load(ba, 0);
  for (int kb = 0; kb < H; kb += 128) {
    load(bb, kb + 64);                                   // H is a multiple of 128
    mul(ba);
    if (kb + 128 < H) load(ba, kb + 128);
    mul(bb);
  }
  const float sc = row_ok ? a.lm_rs[j] : 0.f;
  float best[2] = {-INFINITY, -INFINITY};
  int bidx[2] = {0x7FFFFFFF, 0x7FFFFFFF};
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // accumulator elements 4 q .. 4 q + 3: vocabulary rows 8 q + 4 hf .. + 3 of tile t
      const int vr = v0 + 32 * t + 8 * q + 4 * hf;
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = acc[t][4 * q + e] * sc;
      if (row_ok && a.logits) {
        float* dst = a.logits + (size_t)j * V + vr;
        if (vr + 3 < V) {
          *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) if (vr + e < V) dst[e] = o[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (vr + e < V && (o[e] > best[t >> 1] || (o[e] == best[t >> 1] && vr + e < bidx[t >> 1]))) {
          best[t >> 1] = o[e];
          bidx[t >> 1] = vr + e;
        }
    }
  // each 64-row block: the other half of its rows is in lane l ^ 32
#pragma unroll
  for (int p2 = 0; p2 < 2; ++p2) {
    const float ov = __shfl_xor(best[p2], 32, 64);
    const int oi = __shfl_xor(bidx[p2], 32, 64);
    if (ov > best[p2] || (ov == best[p2] && oi < bidx[p2])) { best[p2] = ov; bidx[p2] = oi; }
    const int blk = (v0 + 64 * p2) / LM_ROWS;
    if (row_ok && hf == 0 && v0 + 64 * p2 < V) {
      a.lm_val[(size_t)j * a.lm_blocks + blk] = best[p2];
      a.lm_idx[(size_t)j * a.lm_blocks + blk] = bidx[p2];
    }
  }
}

// LM head: logits[b][v] = RMSNorm(X_L)[b] . W_lm[v] for 16 vocabulary rows per
// workgroup, plus the block's (max, lowest index) per row for the argmax.
template <typename WT, int NB>
__global__ __launch_bounds__(NT) void lm_head_kernel(Args args) {
  KArgs& a = kernel_args();
  Smem s = make_smem(a);
  constexpr int RPW = rpw_for<NB>();
  constexpr int ROWS = LM_ROWS;
  const int v0 = blockIdx.x * ROWS;
  const int n = min(ROWS, a.V - v0);
  const WT* W = static_cast<const WT*>(a.lm_head);
  Gemv<WT, NB, RPW, (NB > 1)> g{W, W, n, v0, n, a.H};
  Task none{};
  gemv<WT, NB, RPW, (NB > 1)>(a, s, g, a.lm_x, a.M, a.final_norm, true, false, false, none, 0, nullptr, 0);
  for (int e = threadIdx.x; e < n * a.M; e += NT) {
    const int row = e / a.M, b = e - row * a.M;
    if (a.logits) a.logits[(size_t)b * a.V + v0 + row] = s.res[row * NB + b];
  }
  if (threadIdx.x < a.M) {
    const int b = threadIdx.x;
    float best = s.res[b];
    int bi = 0;
    for (int row = 1; row < n; ++row) {
      const float v = s.res[row * NB + b];
      if (v > best) { best = v; bi = row; }
    }
    a.lm_val[(size_t)b * a.lm_blocks + blockIdx.x] = best;
    a.lm_idx[(size_t)b * a.lm_blocks + blockIdx.x] = v0 + bi;
  }
}

// LM head for a few input rows (NB <= 4): the normalised rows sit in shared
// memory and every lane streams its weight slices straight into registers,
// 16 loads of 16 bytes in flight per lane, with many workgroups per compute
// unit (no weight ring), so the vocabulary matrix streams at full bandwidth.
// Wave w of workgroup i owns rows i * LM_ROWS + w * 16 .. + 16; per row a
// lane sums its 8-column slices of every 512-column block, then the wave
// reduces.  Same outputs as lm_head_kernel: logits and the block's (max,
// lowest index) per input row.
constexpr int LMF_RPW = LM_ROWS / NWAVE;      // rows per wave
template <typename WT, int NB>
__global__ __launch_bounds__(NT) void lm_head_regs(Args args) {
  using E = Elem<WT>;
  constexpr int VEC = E::VEC;
  constexpr int RB = 4, UB = 4 / VEC;          // rows x 512-column blocks per batch of loads
  KArgs& a = kernel_args();
  extern __shared__ __align__(16) float lm_smem[];
  float* xs = lm_smem;                         // [NB][H] = x * gain
  float* red = lm_smem + NB * a.H;             // [NWAVE][NB] partial sums, then [NB] scales
  float* bestv = red + NWAVE * NB + NB;        // [NWAVE][NB]
  int* besti = reinterpret_cast<int*>(bestv + NWAVE * NB);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int H = a.H, nb = a.M;
  // stage the normalised input rows
  float ss[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    ss[b] = 0.f;
    if (b >= nb) continue;
    for (int k = t * 4; k < H; k += NT * 4) {
      float4 v = *reinterpret_cast<const float4*>(a.lm_x + (size_t)b * H + k);
      const float4 g = *reinterpret_cast<const float4*>(a.final_norm + k);
      ss[b] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      v.x *= g.x; v.y *= g.y; v.z *= g.z; v.w *= g.w;
      *reinterpret_cast<float4*>(xs + b * H + k) = v;
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float w = wave_sum(ss[b]);
    if (lane == 0) red[wave * NB + b] = w;
  }
  __syncthreads();
  if (t < nb) {
    float tot = 0.f;
    for (int w = 0; w < NWAVE; ++w) tot += red[w * NB + t];
    red[NWAVE * NB + t] = 1.0f / sqrtf(tot / (float)H + a.eps);
  }
  __syncthreads();
  float scale[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) scale[b] = b < nb ? red[NWAVE * NB + b] : 0.f;

  const WT* W = static_cast<const WT*>(a.lm_head);
  const int iters = (H + 511) / 512;
  const int r0 = blockIdx.x * LM_ROWS + wave * LMF_RPW;
  float bv[NB];
  int bi[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) { bv[b] = -INFINITY; bi[b] = 0x7FFFFFFF; }
  for (int jr = 0; jr < LMF_RPW; jr += RB) {
    float acc[RB][NB];
#pragma unroll
    for (int j = 0; j < RB; ++j)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[j][b] = 0.f;
    for (int it0 = 0; it0 < iters; it0 += UB) {
      v4u w[RB][UB][VEC];
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const int row = min(r0 + jr + j, a.V - 1);
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          const int col = (it0 + u) * 512 + lane * 8;
          const v4u* p = reinterpret_cast<const v4u*>(W + (size_t)row * H + min(col, H - 8));
#pragma unroll
          for (int v = 0; v < VEC; ++v) w[j][u][v] = __builtin_nontemporal_load(p + v);
        }
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int col = (it0 + u) * 512 + lane * 8;
        if (col >= H) continue;
        float xv[NB][8];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float4 x0 = *reinterpret_cast<const float4*>(xs + b * H + col);
          const float4 x1 = *reinterpret_cast<const float4*>(xs + b * H + col + 4);
          xv[b][0] = x0.x; xv[b][1] = x0.y; xv[b][2] = x0.z; xv[b][3] = x0.w;
          xv[b][4] = x1.x; xv[b][5] = x1.y; xv[b][6] = x1.z; xv[b][7] = x1.w;
        }
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          float wf[8];
          E::unpack(w[j][u], wf);
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[j][b] = fmaf(wf[e], xv[b][e], acc[j][b]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int row = r0 + jr + j;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float v = wave_sum(acc[j][b]) * scale[b];
        if (b < nb && row < a.V) {
          if (lane == 0 && a.logits) a.logits[(size_t)b * a.V + row] = v;
          if (v > bv[b]) { bv[b] = v; bi[b] = row; }        // rows ascend: the first maximum wins
        }
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b) { bestv[wave * NB + b] = bv[b]; besti[wave * NB + b] = bi[b]; }
  }
  __syncthreads();
  if (t < nb) {
    float best = bestv[t];
    int bidx = besti[t];
    for (int w = 1; w < NWAVE; ++w) {
      const float v = bestv[w * NB + t];
      const int i = besti[w * NB + t];
      if (v > best || (v == best && i < bidx)) { best = v; bidx = i; }
    }
    a.lm_val[(size_t)t * a.lm_blocks + blockIdx.x] = best;
    a.lm_idx[(size_t)t * a.lm_blocks + blockIdx.x] = bidx;
  }
}

// Kernels whose dynamic shared memory exceeds the default limit must opt in,
// once per device.  `granted` holds the bytes granted so far per device; the
// callers hold the library's lock.
constexpr int kMaxDevices = 64;
template <typename K>
inline hipError_t allow_lds(K kernel, uint32_t bytes, uint32_t (&granted)[kMaxDevices]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (bytes <= 64 * 1024 || bytes <= granted[dev]) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) granted[dev] = bytes;
  return e;
}

// A persistent interpreter needs all of its workgroups resident at once (a
// worker waits on tiles other workers produce): refuse a launch of `per_cu`
// workgroups per compute unit that registers or shared memory do not allow.
template <typename K>
inline hipError_t check_resident(K kernel, uint32_t lds_bytes, int per_cu) {
  int fit = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&fit, kernel, NT, lds_bytes);
  if (e != hipSuccess) return e;
  return fit >= per_cu ? hipSuccess : hipErrorCooperativeLaunchTooLarge;
}

#ifdef MK_PREFILL_UNIT
#include "prefill.h"

__device__ __forceinline__ void run_prefill_instr(KArgs& a, Smem& s, const Task in, uint32_t idx, bool mega, int only_op) {
  const int op = only_op ? only_op : in.op;
  switch (op) {
    case mk::OP_P_EMBED: op_p_embed(a, in, idx, mega); break;
    case mk::OP_P_QKV: op_p_qkv(a, s, in, idx, mega); break;
    case mk::OP_P_ATTN: op_p_attn(a, s, in, idx, mega); break;
    case mk::OP_P_OPROJ: op_p_resid(a, s, in, idx, mega, false); break;
    case mk::OP_P_GATEUP: op_p_gateup(a, s, in, idx, mega); break;
    case mk::OP_P_DOWN: op_p_resid(a, s, in, idx, mega, true); break;
    default:
      if (threadIdx.x == 0) record_error(a, ERR_OPCODE, idx, in.op, 0, 0);
      break;
  }
}

// The prefill interpreter (bf16 models): same pop / wait / signal loop over the
// prefill queue's 2-D tiles.
__global__ __launch_bounds__(NT) void mk_interp_prefill(Args args) {
  Smem s = make_smem(kernel_args());
  const uint32_t qi = blockIdx.x % args.n_queues;
  uint32_t k_next = 0;
  if (threadIdx.x == 0) {
    KArgs& a = kernel_args();
    k_next = __hip_atomic_fetch_add(a.heads + qi * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  for (;;) {
    KArgs& a = kernel_args();
    if (threadIdx.x == 0) {
      const uint64_t i = (uint64_t)k_next * a.n_queues + qi;
      const bool go = i < a.n_instr && !aborted(a);
      *s.idx = go ? (uint32_t)i : 0xFFFFFFFFu;
      if (go) k_next = __hip_atomic_fetch_add(a.heads + qi * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const uint32_t idx = __builtin_amdgcn_readfirstlane(*s.idx);
    __syncthreads();
    if (idx == 0xFFFFFFFFu) break;
    unsigned long long t0 = 0;
    if (a.trace) t0 = wall_clock64();
    run_prefill_instr(a, s, load_instr(a, idx), idx, true, 0);
    if (a.trace && threadIdx.x == 0) {
      unsigned long long* rec = a.trace + TRACE_WORDS * (size_t)idx;
      rec[0] = (unsigned long long)blockIdx.x << 32;
      rec[1] = t0;
      rec[5] = wall_clock64();
    }
  }
}

template <int OP>
__global__ __launch_bounds__(NT) void kpo_prefill(Args args, uint32_t first) {
  KArgs& a = kernel_args();
  Smem s = make_smem(a);
  const uint32_t idx = first + blockIdx.x;
  const Task in = load_instr(a, idx);
  if (in.op != (OP == KPO_OPROJ_FUSED ? mk::OP_OPROJ : OP)) {
    if (threadIdx.x == 0) record_error(a, ERR_OPCODE, idx, in.op, 0, 0);
    return;
  }
  run_prefill_instr(a, s, in, idx, false, OP);
}

struct PrefillLaunch {
  // Everything that can refuse a call, before anything is enqueued.
  static hipError_t prep(const Args& a, int exec_mode, int per_cu) {
    if (exec_mode == MK_MEGAKERNEL) {
      static uint32_t granted[kMaxDevices] = {};
      hipError_t e = allow_lds(mk_interp_prefill, a.lds_bytes, granted);
      return e == hipSuccess ? check_resident(mk_interp_prefill, a.lds_bytes, per_cu) : e;
    }
    static uint32_t granted[mk::OP_COUNT][kMaxDevices] = {};
    hipError_t e = hipSuccess;
#define PREP_CASE(OPC) if (e == hipSuccess) e = allow_lds(kpo_prefill<OPC>, a.lds_bytes, granted[OPC]);
    PREP_CASE(mk::OP_P_EMBED) PREP_CASE(mk::OP_P_QKV) PREP_CASE(mk::OP_P_ATTN) PREP_CASE(mk::OP_P_OPROJ)
    PREP_CASE(mk::OP_P_GATEUP) PREP_CASE(mk::OP_P_DOWN)
#undef PREP_CASE
    return e;
  }
  static hipError_t mega(const Args& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL(mk_interp_prefill, dim3(grid), dim3(NT), a.lds_bytes, st, a);
    return hipGetLastError();
  }
  static hipError_t kpo(const Args& a, uint32_t op, uint32_t first, uint32_t count, hipStream_t st) {
    switch (op) {
#define KPO_CASE(OPC)                                                                              \
      case OPC:                                                                                    \
        hipLaunchKernelGGL((kpo_prefill<OPC>), dim3(count), dim3(NT), a.lds_bytes, st, a, first);  \
        break;
      KPO_CASE(mk::OP_P_EMBED) KPO_CASE(mk::OP_P_QKV) KPO_CASE(mk::OP_P_ATTN) KPO_CASE(mk::OP_P_OPROJ)
      KPO_CASE(mk::OP_P_GATEUP) KPO_CASE(mk::OP_P_DOWN)
#undef KPO_CASE
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
};

#endif  // MK_PREFILL_UNIT

// Execution modes of the preparation step beyond the public ones: the
// multi-step interpreter and the multi-stream kernels.
constexpr int kLoopMode = 100;
constexpr int kMultiStreamMode = 101;

template <typename WT, int NB>
struct Launch {
  // The multi-step interpreter is built for bf16 models (those with an
  // embedding and an LM head here); for fp32 ones the entry point refuses.
  static constexpr bool kHasLoop = sizeof(WT) == 2;
  // Everything that can refuse a call, before anything is enqueued: the shared
  // memory opt-in of every kernel the call may launch and, for the megakernel,
  // that all of its workgroups can be resident at once (for the multi-stream
  // kernels: that `per_cu` workgroups of each fit on one compute unit, so that
  // any `per_cu` of them, from whichever kernels, fit together).
  static hipError_t prep(const Args& a, int exec_mode, int per_cu) {
    if (exec_mode == MK_MEGAKERNEL) {
      if (a.attn_pop) {
        static uint32_t granted[kMaxDevices] = {};
        hipError_t e = allow_lds(mk_interp<WT, NB, false, true>, a.lds_bytes, granted);
        return e == hipSuccess ? check_resident(mk_interp<WT, NB, false, true>, a.lds_bytes, per_cu) : e;
      }
      static uint32_t granted[kMaxDevices] = {};
      hipError_t e = allow_lds(mk_interp<WT, NB>, a.lds_bytes, granted);
      return e == hipSuccess ? check_resident(mk_interp<WT, NB>, a.lds_bytes, per_cu) : e;
    }
    if (exec_mode == kMultiStreamMode) {
      static uint32_t granted_ms[KPO_OPROJ_FUSED + 1][kMaxDevices] = {};
      hipError_t e = hipSuccess;
#define PREP_MS(OPC)                                                                                \
      if (e == hipSuccess) e = allow_lds(ms_kernel<WT, NB, OPC>, a.lds_bytes, granted_ms[OPC]);      \
      if (e == hipSuccess) e = check_resident(ms_kernel<WT, NB, OPC>, a.lds_bytes, per_cu);
      PREP_MS(mk::OP_EMBED) PREP_MS(mk::OP_QKV) PREP_MS(mk::OP_ATTN) PREP_MS(mk::OP_COMBINE)
      PREP_MS(mk::OP_OPROJ) PREP_MS(mk::OP_GATEUP) PREP_MS(mk::OP_DOWN) PREP_MS(KPO_OPROJ_FUSED)
#undef PREP_MS
      return e;
    }
    if (exec_mode == kLoopMode) {
      if constexpr (kHasLoop) {
        static uint32_t granted[kMaxDevices] = {};
        hipError_t e = allow_lds(mk_interp<WT, NB, true>, a.lds_bytes, granted);
        return e == hipSuccess ? check_resident(mk_interp<WT, NB, true>, a.lds_bytes, per_cu) : e;
      }
      return hipErrorInvalidValue;
    }
    static uint32_t granted[KPO_OPROJ_FUSED + 1][kMaxDevices] = {};
    hipError_t e = hipSuccess;
#define PREP_CASE(OPC) if (e == hipSuccess) e = allow_lds(kpo_kernel<WT, NB, OPC>, a.lds_bytes, granted[OPC]);
    PREP_CASE(mk::OP_EMBED) PREP_CASE(mk::OP_QKV) PREP_CASE(mk::OP_ATTN) PREP_CASE(mk::OP_COMBINE)
    PREP_CASE(mk::OP_OPROJ) PREP_CASE(mk::OP_GATEUP) PREP_CASE(mk::OP_DOWN) PREP_CASE(KPO_OPROJ_FUSED)
#undef PREP_CASE
    return e;
  }
  static hipError_t mega(const Args& a, int grid, hipStream_t st) {
    if (a.attn_pop)      // splits handed out at run time (a variant of its own: the default path's code is untouched)
      hipLaunchKernelGGL((mk_interp<WT, NB, false, true>), dim3(grid), dim3(NT), a.lds_bytes, st, a);
    else
      hipLaunchKernelGGL((mk_interp<WT, NB>), dim3(grid), dim3(NT), a.lds_bytes, st, a);
    return hipGetLastError();
  }
  // Persistent multi-step decode: the interpreter over a loop queue, a.steps times.
  static hipError_t loop(const Args& a, int grid, hipStream_t st) {
    if constexpr (kHasLoop) {
      hipLaunchKernelGGL((mk_interp<WT, NB, true>), dim3(grid), dim3(NT), a.lds_bytes, st, a);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  // One segment of the multi-stream mode: `grid` workgroups stride over its instructions.
  static hipError_t ms(const Args& a, uint32_t op, uint32_t first, uint32_t count, uint32_t grid, hipStream_t st) {
    if (op == mk::OP_OPROJ && a.fuse_combine) op = KPO_OPROJ_FUSED;
    switch (op) {
#define MS_CASE(OPC)                                                                               \
      case OPC:                                                                                    \
        hipLaunchKernelGGL((ms_kernel<WT, NB, OPC>), dim3(grid), dim3(NT), a.lds_bytes, st, a, first, count); \
        break;
      MS_CASE(mk::OP_EMBED) MS_CASE(mk::OP_QKV) MS_CASE(mk::OP_ATTN) MS_CASE(mk::OP_COMBINE)
      MS_CASE(mk::OP_OPROJ) MS_CASE(mk::OP_GATEUP) MS_CASE(mk::OP_DOWN) MS_CASE(KPO_OPROJ_FUSED)
#undef MS_CASE
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  static hipError_t kpo(const Args& a, uint32_t op, uint32_t first, uint32_t count, hipStream_t st) {
    if (op == mk::OP_OPROJ && a.fuse_combine) op = KPO_OPROJ_FUSED;
    switch (op) {
#define KPO_CASE(OPC)                                                                              \
      case OPC:                                                                                    \
        hipLaunchKernelGGL((kpo_kernel<WT, NB, OPC>), dim3(count), dim3(NT), a.lds_bytes, st, a, first); \
        break;
      KPO_CASE(mk::OP_EMBED) KPO_CASE(mk::OP_QKV) KPO_CASE(mk::OP_ATTN) KPO_CASE(mk::OP_COMBINE)
      KPO_CASE(mk::OP_OPROJ) KPO_CASE(mk::OP_GATEUP) KPO_CASE(mk::OP_DOWN) KPO_CASE(KPO_OPROJ_FUSED)
#undef KPO_CASE
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  // The LM head's kernel and its shared memory: for up to 4 rows the register
  // streaming kernel (normalised rows + per-wave partials) where they fit in
  // 64 KB, else for bf16 weights the matrix cores, else the ring GEMV.
  static bool lm_regs(const Args& a) {
    return NB <= 4 && a.H % 8 == 0 && 4u * (NB * a.H + NWAVE * NB + NB + 2 * NWAVE * NB) <= 64 * 1024;
  }
  static hipError_t prep_lm(const Args& a) {
    if (lm_regs(a) || lm_mfma(a)) return hipSuccess;
    static uint32_t granted[kMaxDevices] = {};
    return allow_lds(lm_head_kernel<WT, NB>, a.lds_bytes, granted);
  }
  // 2 to 32 rows of bf16 weights: the matrix-core LM head (H a multiple of 128)
  static bool lm_mfma(const Args& a) {
    return sizeof(WT) == 2 && a.M >= 2 && a.M <= 32 && a.H % 128 == 0 && a.lm_y && a.lm_rs;
  }
  static hipError_t lm(const Args& a, hipStream_t st) {
    if (lm_regs(a)) {
      const uint32_t bytes = 4u * (NB * a.H + NWAVE * NB + NB + 2 * NWAVE * NB);
      hipLaunchKernelGGL((lm_head_regs<WT, NB>), dim3(a.lm_blocks), dim3(NT), bytes, st, a);
    } else if (lm_mfma(a)) {
      if constexpr (sizeof(WT) == 2) {
        hipLaunchKernelGGL((lm_prep_kernel<WT>), dim3(a.M), dim3(NT), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((lm_head_mfma<WT>), dim3((a.V + LMM_ROWS - 1) / LMM_ROWS), dim3(NT), 0, st, a);
      }
    } else {
      hipLaunchKernelGGL((lm_head_kernel<WT, NB>), dim3(a.lm_blocks), dim3(NT), a.lds_bytes, st, a);
    }
    return hipGetLastError();
  }
};

struct Table {
  hipError_t (*prep)(const Args&, int exec_mode, int per_cu);
  hipError_t (*mega)(const Args&, int grid, hipStream_t);
  hipError_t (*loop)(const Args&, int grid, hipStream_t);
  hipError_t (*kpo)(const Args&, uint32_t op, uint32_t first, uint32_t count, hipStream_t);
  hipError_t (*ms)(const Args&, uint32_t op, uint32_t first, uint32_t count, uint32_t grid, hipStream_t);
  hipError_t (*prep_lm)(const Args&);
  hipError_t (*lm)(const Args&, hipStream_t);
};


}  // namespace mkd
