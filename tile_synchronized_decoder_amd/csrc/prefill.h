// Prefill op bodies for gfx950: 128 x 128 MFMA GEMM tiles with fused RMSNorm
// scale, QK-norm, RoPE, KV-cache write, SwiGLU and residual epilogues, and a
// causal flash-attention tile (128 query rows x one head) on MFMA.
//
// Same queue discipline as decode (MegaOps abstract: tile-granular
// dependencies; lecture summary: symbolic sequence length S): the queue is
// built for S_max, row blocks at or past the runtime length are no-ops that
// still signal, and the attention tile of row block m waits only on the
// key / value tiles of row blocks <= m.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, wave64): operand A supplies
// rows i = lane % 32 with k = 8 * (lane / 32) .. + 8, operand B columns
// j = lane % 32 with the same k; accumulator element v of a lane sits at row
// 8 * (v / 4) + 4 * (lane / 32) + v % 4, column lane % 32.  A 128 x 128 tile
// is 2 x 2 waves of 64 x 64, each 2 x 2 MFMA blocks.  LDS rows of 64 bf16
// (128 B) hold 8 chunks of 16 B stored at chunk ^ (row & 7), so the 32 rows
// a matrix operand read touches spread over the banks.
#pragma once

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int PBM = 128;        // rows of a prefill tile
constexpr int PBN = 128;        // output columns of a prefill GEMM tile (one head for QKV)
constexpr int PKS = 64;         // K step (one 128-byte bf16 row chunk set)
constexpr int PKB = 64;         // keys per attention block

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

__device__ __forceinline__ bf16x8 as_bf16x8(v4u v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// One chunk (8 consecutive k) of an operand row from a swizzled 128-byte-row tile.
__device__ __forceinline__ bf16x8 ld_frag(const uint8_t* tile, int row, int chunk) {
  return as_bf16x8(*reinterpret_cast<const v4u*>(tile + row * 128 + swz(row, chunk) * 16));
}

// Device-coherent 16-byte load and 4-byte store: the KV-cache rows that the
// QKV tiles write are read back by attention tiles on other compute units (and
// other XCDs, whose L2 caches are not coherent with each other) in the same
// launch, so they travel like the fp32 activation tiles.
__device__ __forceinline__ v4u ld_cg_v4u(const void* p) {
  uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<void*>(p));
  const uint64_t x = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t y = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v4u{(uint32_t)x, (uint32_t)(x >> 32), (uint32_t)y, (uint32_t)(y >> 32)};
}
__device__ __forceinline__ void st_cg_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Activation tiles (X, QKV, ATT, HRES, ACT) are read with ordinary L2-cached
// loads, so the many column tiles of one row block share them through L2
// instead of each fetching them from memory.  This is safe because every
// 128-byte line of these tensors is written by exactly one producer tile
// (column tiles are 128 floats wide, rows a multiple of 64 floats), with
// device-coherent stores, and is first read on any XCD only after that
// tile's barrier was observed; no L2 holds a copy from before the launch
// (caches are written back and invalidated at kernel boundaries).
__device__ __forceinline__ float4 ld_act4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float ld_act(const float* p) { return *p; }

// Rotary cos / sin of position `pos` and pair index i, angle reduced in float64.
__device__ __forceinline__ void rope_cs(KArgs& a, int pos, int i, float& c, float& s) {
  const double ang = (double)pos * a.rope_inv[i];
  const double k = rint(ang * 0.15915494309189535);
  const double red = fma(-k, 6.283185307179586, ang) - k * 2.4492935982947064e-16;
  sincosf((float)red, &s, &c);
}

// ---------------------------------------------------------------------------- GEMM tile

struct PGemm {
  const float* x;          // A rows (fp32 workspace), leading dimension K
  const float* gain;       // RMSNorm gain applied to A (nullable)
  bool norm;               // scale each output row by RMSNorm(A row)
  const uint16_t* w0;      // weight rows for the first 128 columns
  const uint16_t* w1;      // second matrix (gate/up: up rows), or null
  int n0, n_total;         // first output column; rows of the weight matrix
  int K;
  int r0, rows;            // first A row of the tile; valid rows (< PBM)
};

struct PAcc { f32x16 c[2][2]; };

// Issue the weight DMA of K step ks into LDS tile b (128 or 256 rows of 128 B).
__device__ __forceinline__ void p_issue_b(const PGemm& g, uint8_t* b, int ks, int wave, int lane) {
  const int nrow = g.w1 ? 2 * PBN : PBN;
  for (int d = wave; d < nrow / 8; d += NWAVE) {
    const int row = d * 8 + lane / 8;
    const int c = (lane % 8) ^ (row & 7);
    const int half = row / PBN;
    int wr = g.n0 + (row % PBN);
    if (wr >= g.n_total) wr = g.n_total - 1;
    const uint16_t* src = (half ? g.w1 : g.w0) + (size_t)wr * g.K + ks * PKS + c * 8;
    dma_lds16<0>(src, b + d * 1024);
  }
}

// Activation operand of K step ks: this thread's 32 floats of one row (rows
// past the tile read as zeros).  The loads are only issued here; p_store_a
// consumes them, so they overlap the matrix-core work of the current step.
struct PARegs { float4 v[8]; };

__device__ __forceinline__ void p_load_a(const PGemm& g, int ks, PARegs& r) {
  const int t = threadIdx.x, row = t >> 1, half = t & 1;
  const int k0 = ks * PKS + half * 32;
  if (row < g.rows) {
    const float* src = g.x + (size_t)(g.r0 + row) * g.K + k0;
#pragma unroll
    for (int q = 0; q < 8; ++q) r.v[q] = ld_act4(src + 4 * q);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) r.v[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Sum of squares (RMSNorm), gain, bf16 rounding, swizzled store into LDS.
__device__ __forceinline__ void p_store_a(const PGemm& g, int ks, uint8_t* a, PARegs& r, float& ss) {
  const int t = threadIdx.x, row = t >> 1, half = t & 1;
  const int k0 = ks * PKS + half * 32;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    ss += r.v[q].x * r.v[q].x + r.v[q].y * r.v[q].y + r.v[q].z * r.v[q].z + r.v[q].w * r.v[q].w;
    if (g.gain) {
      const float4 gg = *reinterpret_cast<const float4*>(g.gain + k0 + 4 * q);
      r.v[q].x *= gg.x; r.v[q].y *= gg.y; r.v[q].z *= gg.z; r.v[q].w *= gg.w;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 u = r.v[2 * q], w = r.v[2 * q + 1];
    v4u pk = {pack_bf16(u.x, u.y), pack_bf16(u.z, u.w), pack_bf16(w.x, w.y), pack_bf16(w.z, w.w)};
    *reinterpret_cast<v4u*>(a + row * 128 + swz(row, half * 4 + q) * 16) = pk;
  }
}

__device__ __forceinline__ void p_mfma_step(const uint8_t* a, const uint8_t* b, PAcc& acc, PAcc* acc_up,
                                            int wm, int wn, int lane) {
#pragma unroll
  for (int kk = 0; kk < PKS / 16; ++kk) {
    const int chunk = kk * 2 + (lane >> 5);
    bf16x8 af[2], bfr[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) af[mi] = ld_frag(a, wm * 64 + mi * 32 + (lane & 31), chunk);
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) bfr[ni] = ld_frag(b, wn * 64 + ni * 32 + (lane & 31), chunk);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        acc.c[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc.c[mi][ni], 0, 0, 0);
    if (acc_up) {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) bfr[ni] = ld_frag(b, PBN + wn * 64 + ni * 32 + (lane & 31), chunk);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc_up->c[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc_up->c[mi][ni], 0, 0, 0);
    }
  }
}

// LDS of a GEMM tile: two activation stages, three weight stages, then the
// row statistics ([NT] partial sums, then [PBM] row scales).
constexpr int P_BSTAGES = 3;
__device__ __forceinline__ float* p_row_stats(Smem& s, bool two_mats) {
  return reinterpret_cast<float*>(s.ring + 2 * PBM * 128 + P_BSTAGES * (two_mats ? 2 : 1) * PBN * 128);
}

// Full K loop of one tile.  Weights are DMA'd two K steps ahead (three
// stages), activations one step ahead through registers; the loads of the
// next steps are in flight while the current step runs on the matrix cores.
// The first two weight steps are issued before the tile waits (`mega`).
// Leaves the row scales (RMSNorm factors, or 1) in p_row_stats()[NT ..].
__device__ __forceinline__ bool p_gemm(KArgs& a, Smem& s, const PGemm& g, PAcc& acc, PAcc* acc_up, bool mega,
                                       const Instr in, uint32_t idx) {
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const bool two = g.w1 != nullptr;
  const int bbytes = (two ? 2 : 1) * PBN * 128;
  uint8_t* abase = s.ring;                               // two activation stages
  uint8_t* bbase = s.ring + 2 * PBM * 128;
  float* rs = p_row_stats(s, two);
  const int nks = g.K / PKS;

  p_issue_b(g, bbase, 0, wave, lane);
  if (nks > 1) p_issue_b(g, bbase + bbytes, 1, wave, lane);
  if (mega && !wait_tiles(a, in, idx)) { wait_vm<0>(); return false; }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      acc.c[mi][ni] = (f32x16){};
      if (acc_up) acc_up->c[mi][ni] = (f32x16){};
    }
  float ss = 0.f;
  PARegs ar;
  p_load_a(g, 0, ar);
  wait_vm<0>();
  p_store_a(g, 0, abase, ar, ss);
  __syncthreads();
  int bcur = 0;                                          // stage of step ks
  for (int ks = 0; ks < nks; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < nks, more2 = ks + 2 < nks;
    if (more) p_load_a(g, ks + 1, ar);
    const int b2 = bcur + 2 >= P_BSTAGES ? bcur + 2 - P_BSTAGES : bcur + 2;
    if (more2) p_issue_b(g, bbase + b2 * bbytes, ks + 2, wave, lane);
    p_mfma_step(abase + cur * (PBM * 128), bbase + bcur * bbytes, acc, acc_up, wm, wn, lane);
    if (more) {
      // the activations of step ks + 1 (issued before the weights of step ks + 2) and the
      // weights of step ks + 1 (issued a step earlier) have landed once only the weight
      // loads of step ks + 2 may still be outstanding
      if (!more2) wait_vm<0>();
      else if (two) wait_vm<2 * PBN / 8 / NWAVE>();
      else wait_vm<PBN / 8 / NWAVE>();
      p_store_a(g, ks + 1, abase + (cur ^ 1) * (PBM * 128), ar, ss);
    }
    __syncthreads();
    bcur = bcur + 1 == P_BSTAGES ? 0 : bcur + 1;
  }
  if (mega) trace_mark(a, idx, 4);
  // row scales: each row's two threads hold halves of sum(x^2)
  rs[t] = ss;
  __syncthreads();
  if (t < PBM) {
    const float tot = rs[2 * t] + rs[2 * t + 1];
    rs[NT + t] = g.norm ? 1.0f / sqrtf(tot / (float)g.K + a.eps) : 1.0f;
  }
  __syncthreads();
  return true;
}

// Element (row, col) of accumulator value v of block (mi, ni) of wave (wm, wn).
__device__ __forceinline__ int p_row(int wm, int mi, int v, int lane) { return wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }
__device__ __forceinline__ int p_col(int wn, int ni, int lane) { return wn * 64 + ni * 32 + (lane & 31); }

__device__ __forceinline__ bool p_block_live(KArgs& a, int m) { return m * PBM < a.seq_len; }

// P_EMBED(m): X_0 rows of block m = embedding rows of their tokens.
__device__ __forceinline__ void op_p_embed(KArgs& a, const Instr in, uint32_t idx, bool mega) {
  const int m = in.a0;
  const uint16_t* E = static_cast<const uint16_t*>(a.embed);
  const int r0 = m * PBM, rows = max(0, min(PBM, a.seq_len - r0));
  for (int e = threadIdx.x; e < rows * a.H; e += NT) {
    const int row = e / a.H, c = e - row * a.H;
    const int tok = a.tokens[r0 + row];
    float v = 0.f;
    if (tok < 0 || tok >= a.V) {
      if (c == 0) record_error(a, ERR_TOKEN, idx, (uint32_t)(r0 + row), (uint32_t)tok, (uint32_t)a.V);
    } else {
      v = bf16_to_f32(E[(size_t)tok * a.H + c]);
    }
    st_cg(a.X + (size_t)(r0 + row) * a.H + c, v);
  }
  if (mega) signal_tile(a, in);
}

// P_QKV(m, n0, n1): one head's columns of QKV for row block m, with the
// RMSNorm row scale, QK-norm and RoPE (q, k), the KV-cache write (k, v).
__device__ __forceinline__ void op_p_qkv(KArgs& a, Smem& s, const Instr in, uint32_t idx, bool mega) {
  const int l = in.layer, m = in.a0, n0 = in.a1;
  if (!p_block_live(a, m)) {
    if (mega && wait_tiles(a, in, idx)) signal_tile(a, in);
    return;
  }
  const int r0 = m * PBM, rows = min(PBM, a.seq_len - r0);
  PGemm g{a.X + l * a.sX, a.attn_norm + (size_t)l * a.H, true,
          static_cast<const uint16_t*>(a.wqkv) + (size_t)l * a.NQKV * a.H, nullptr, n0, a.NQKV, a.H, r0, rows};
  PAcc acc;
  if (!p_gemm(a, s, g, acc, nullptr, mega, in, idx)) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, wm = wave >> 1, wn = wave & 1;
  const float* rs = p_row_stats(s, false) + NT;
  // stage the scaled tile (fp32 [128][128]) over the operand buffers
  float* ct = reinterpret_cast<float*>(s.ring);
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = p_row(wm, mi, v, lane), col = p_col(wn, ni, lane);
        ct[row * PBN + col] = acc.c[mi][ni][v] * rs[row];
      }
  __syncthreads();
  const int hh = n0 / PBN;                        // head index within [q | k | v]
  const bool is_q = hh < a.nq, is_k = !is_q && hh < a.nq + a.nkv;
  const int row = t >> 1, part = t & 1;           // two threads per row: pairs [part*32, part*32+32)
  const int HALF = PBN / 2;
  float x0[32], x1[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) { x0[k] = ct[row * PBN + part * 32 + k]; x1[k] = ct[row * PBN + HALF + part * 32 + k]; }
  if ((is_q || is_k) && a.qk_norm) {
    float ssq = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) ssq += x0[k] * x0[k] + x1[k] * x1[k];
    ssq += __shfl_xor(ssq, 1, 64);
    const float sc = 1.0f / sqrtf(ssq / (float)PBN + a.eps);
    const float* gn = (is_q ? a.q_norm : a.k_norm) + (size_t)l * PBN;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      x0[k] = x0[k] * sc * gn[part * 32 + k];
      x1[k] = x1[k] * sc * gn[HALF + part * 32 + k];
    }
  }
  const int pos = r0 + row;
  if (is_q || is_k) {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      float c, sn;
      rope_cs(a, pos, part * 32 + k, c, sn);
      const float y0 = x0[k] * c - x1[k] * sn, y1 = x1[k] * c + x0[k] * sn;
      x0[k] = y0; x1[k] = y1;
    }
  }
  if (row < rows) {
    float* out = a.QKV + l * a.sQKV + (size_t)pos * a.NQKV + n0;
#pragma unroll
    for (int k = 0; k < 32; ++k) { st_cg(out + part * 32 + k, x0[k]); st_cg(out + HALF + part * 32 + k, x1[k]); }
    if (!is_q) {
      const int gidx = hh - a.nq - (is_k ? 0 : a.nkv);
      uint16_t* cache = static_cast<uint16_t*>(is_k ? a.kc : a.vc) +
                        ((((size_t)l * a.M_cache + a.kv_row) * a.nkv + gidx) * a.ctx_max + pos) * PBN;
      uint32_t* c0 = reinterpret_cast<uint32_t*>(cache + part * 32);
      uint32_t* c1 = reinterpret_cast<uint32_t*>(cache + HALF + part * 32);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        st_cg_u32(c0 + k, pack_bf16(x0[2 * k], x0[2 * k + 1]));
        st_cg_u32(c1 + k, pack_bf16(x1[2 * k], x1[2 * k + 1]));
      }
    }
  }
  if (mega) signal_tile(a, in);
}

// P_OPROJ / P_DOWN: out = residual + A W^T (A = ATT_l / ACT_l; residual = X_l / HRES_l).
__device__ __forceinline__ void op_p_resid(KArgs& a, Smem& s, const Instr in, uint32_t idx, bool mega, bool down) {
  const int l = in.layer, m = in.a0, n0 = in.a1;
  if (!p_block_live(a, m)) {
    if (mega && wait_tiles(a, in, idx)) signal_tile(a, in);
    return;
  }
  const int r0 = m * PBM, rows = min(PBM, a.seq_len - r0);
  const int K = down ? a.F : a.NA;
  PGemm g{down ? a.ACT + l * a.sACT : a.ATT + l * a.sATT, nullptr, false,
          static_cast<const uint16_t*>(down ? a.wdown : a.wo) + (size_t)l * a.H * K, nullptr, n0, a.H, K, r0, rows};
  PAcc acc;
  if (!p_gemm(a, s, g, acc, nullptr, mega, in, idx)) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, wm = wave >> 1, wn = wave & 1;
  const float* res = down ? a.HRES + l * a.sHRES : a.X + l * a.sX;
  float* out = down ? a.X + (l + 1) * a.sX : a.HRES + l * a.sHRES;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = p_row(wm, mi, v, lane), col = n0 + p_col(wn, ni, lane);
        if (row < rows && col < a.H) {
          const size_t o = (size_t)(r0 + row) * a.H + col;
          st_cg(out + o, ld_act(res + o) + acc.c[mi][ni][v]);
        }
      }
  if (mega) signal_tile(a, in);
}

// P_GATEUP: ACT = silu(RMSNorm(H) Wg^T) * (RMSNorm(H) Wu^T) for 128 columns.
__device__ __forceinline__ void op_p_gateup(KArgs& a, Smem& s, const Instr in, uint32_t idx, bool mega) {
  const int l = in.layer, m = in.a0, n0 = in.a1;
  if (!p_block_live(a, m)) {
    if (mega && wait_tiles(a, in, idx)) signal_tile(a, in);
    return;
  }
  const int r0 = m * PBM, rows = min(PBM, a.seq_len - r0);
  PGemm g{a.HRES + l * a.sHRES, a.ffn_norm + (size_t)l * a.H, true,
          static_cast<const uint16_t*>(a.wgate) + (size_t)l * a.F * a.H,
          static_cast<const uint16_t*>(a.wup) + (size_t)l * a.F * a.H, n0, a.F, a.H, r0, rows};
  PAcc acc, up;
  if (!p_gemm(a, s, g, acc, &up, mega, in, idx)) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, wm = wave >> 1, wn = wave & 1;
  const float* rs = p_row_stats(s, true) + NT;
  float* out = a.ACT + l * a.sACT;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = p_row(wm, mi, v, lane), col = n0 + p_col(wn, ni, lane);
        if (row < rows && col < a.F) {
          const float gt = acc.c[mi][ni][v] * rs[row], u = up.c[mi][ni][v] * rs[row];
          st_cg(out + (size_t)(r0 + row) * a.F + col, gt / (1.0f + expf(-gt)) * u);
        }
      }
  if (mega) signal_tile(a, in);
}

// ---------------------------------------------------------------------------- causal attention tile

// P_ATTN(m, h): rows of block m attend causally to keys 0 .. last row of the
// block, read back from the KV cache (bf16) that the QKV tiles wrote.
// Shared memory: Q [128][128] bf16 (32 KB, 2 chunk-sets of 64 dims),
// K block [64][128] (16 KB), V^T block [128 dims][64 keys] (16 KB),
// S [128][64] fp32 (32 KB), P [128][64] bf16 (16 KB), row statistics.
__device__ __forceinline__ void op_p_attn(KArgs& a, Smem& s, const Instr in, uint32_t idx, bool mega) {
  constexpr int HD = PBN;
  const int l = in.layer, m = in.a0, h = in.a1;
  const int g = h / a.r;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  if (!p_block_live(a, m)) {
    if (mega && wait_tiles(a, in, idx)) signal_tile(a, in);
    return;
  }
  if (mega && !wait_tiles(a, in, idx)) return;
  const int r0 = m * PBM, rows = min(PBM, a.seq_len - r0);
  uint8_t* qs = s.ring;                                  // [2][128 rows][128 B]
  uint8_t* ks = qs + 2 * PBM * 128;                      // [2][64 keys][128 B]
  uint8_t* vt = ks + 2 * PKB * 128;                      // [128 dims][64 keys] bf16, 128 B rows
  float* sm = reinterpret_cast<float*>(vt + HD * PKB * 2);   // [128][64]
  uint8_t* pb = reinterpret_cast<uint8_t*>(sm + PBM * PKB);  // [128][64] bf16, 128 B rows
  float* mrow = reinterpret_cast<float*>(pb + PBM * PKB * 2);
  float* lrow = mrow + PBM;
  float* arow = lrow + PBM;
  const float scale = 1.0f / sqrtf((float)HD);

  // Q rows (fp32 post-RoPE) -> bf16, two 64-dim halves
  {
    const int row = t >> 1, half = t & 1;
    const float* src = a.QKV + l * a.sQKV + (size_t)(r0 + row) * a.NQKV + h * HD + half * 64;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f), w = u;
      if (row < rows) { u = ld_act4(src + 8 * q); w = ld_act4(src + 8 * q + 4); }
      v4u pk = {pack_bf16(u.x, u.y), pack_bf16(u.z, u.w), pack_bf16(w.x, w.y), pack_bf16(w.z, w.w)};
      *reinterpret_cast<v4u*>(qs + half * PBM * 128 + row * 128 + swz(row, q) * 16) = pk;
    }
  }
  if (t < PBM) { mrow[t] = -INFINITY; lrow[t] = 0.f; }
  PAcc o;                                                // O [128][128]: rows wm*64.., dims wn*64..
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) o.c[mi][ni] = (f32x16){};
  const size_t cache_rows = (((size_t)l * a.M_cache + a.kv_row) * a.nkv + g) * a.ctx_max;
  const uint16_t* Kc = static_cast<const uint16_t*>(a.kc) + cache_rows * HD;
  const uint16_t* Vc = static_cast<const uint16_t*>(a.vc) + cache_rows * HD;
  const int nkeys = r0 + rows;                           // causal: keys 0 .. last row
  for (int k0 = 0; k0 < nkeys; k0 += PKB) {
    __syncthreads();
    // K block: 64 keys x 128 dims as two 64-dim halves (DMA, swizzled)
    for (int d = wave; d < 2 * PKB / 8; d += NWAVE) {     // 16 DMA lines of 1 KB
      const int half = d / (PKB / 8), key = (d % (PKB / 8)) * 8 + lane / 8;
      const int c = (lane % 8) ^ (key & 7);
      const int kk = min(k0 + key, nkeys - 1);
      dma_lds16<1>(Kc + (size_t)kk * HD + half * 64 + c * 8, ks + d * 1024);
    }
    // V block transposed: thread t reads 8 dims of one key and scatters them
    for (int e = t; e < PKB * (HD / 8); e += NT) {
      const int key = e / (HD / 8), d8 = (e % (HD / 8)) * 8;
      const int kk = min(k0 + key, nkeys - 1);
      const v4u v = ld_cg_v4u(Vc + (size_t)kk * HD + d8);
      const uint16_t* hv = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int dim = d8 + j;
        *reinterpret_cast<uint16_t*>(vt + dim * 128 + swz(dim, key / 8) * 16 + (key % 8) * 2) = hv[j];
      }
    }
    wait_vm<0>();
    __syncthreads();
    // S = Q K^T: [128 rows][64 keys]; wave (wm, wn) computes rows wm*64.., keys wn*32..
    {
      f32x16 sc[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
      for (int kk = 0; kk < HD / 16; ++kk) {
        const int half = kk / 4, chunk = (kk % 4) * 2 + (lane >> 5);
        const bf16x8 bfr = ld_frag(ks + half * PKB * 128, wn * 32 + (lane & 31), chunk);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          sc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              ld_frag(qs + half * PBM * 128, wm * 64 + mi * 32 + (lane & 31), chunk), bfr, sc[mi], 0, 0, 0);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = p_row(wm, mi, v, lane), key = wn * 32 + (lane & 31);
          const bool ok = k0 + key <= r0 + row && k0 + key < nkeys;
          sm[row * PKB + key] = ok ? sc[mi][v] * scale : -INFINITY;
        }
    }
    __syncthreads();
    // online softmax per row: two threads per row, 32 keys each
    {
      const int row = t >> 1, half = t & 1;
      float mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < 32; ++k) mx = fmaxf(mx, sm[row * PKB + half * 32 + k]);
      mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
      const float mold = mrow[row];
      const float mnew = fmaxf(mold, mx);
      float sum = 0.f;
      uint32_t pk[16];
#pragma unroll
      for (int k = 0; k < 32; k += 2) {
        const float p0 = mnew == -INFINITY ? 0.f : expf(sm[row * PKB + half * 32 + k] - mnew);
        const float p1 = mnew == -INFINITY ? 0.f : expf(sm[row * PKB + half * 32 + k + 1] - mnew);
        sum += p0 + p1;
        pk[k / 2] = pack_bf16(p0, p1);
      }
      sum += __shfl_xor(sum, 1, 64);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v4u v = {pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]};
        *reinterpret_cast<v4u*>(pb + row * 128 + swz(row, half * 4 + q) * 16) = v;
      }
      __syncthreads();
      if (half == 0) {
        const float al = mold == -INFINITY ? 0.f : expf(mold - mnew);
        arow[row] = al;
        lrow[row] = lrow[row] * al + sum;
        mrow[row] = mnew;
      }
    }
    __syncthreads();
    // O = O * alpha + P V: A = P [128 rows][64 keys], B = V^T [128 dims][64 keys]
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float al = arow[p_row(wm, mi, v, lane)];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) o.c[mi][ni][v] *= al;
      }
#pragma unroll
    for (int kk = 0; kk < PKB / 16; ++kk) {
      const int chunk = kk * 2 + (lane >> 5);
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) af[mi] = ld_frag(pb, wm * 64 + mi * 32 + (lane & 31), chunk);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) bfr[ni] = ld_frag(vt, wn * 64 + ni * 32 + (lane & 31), chunk);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          o.c[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], o.c[mi][ni], 0, 0, 0);
    }
  }
  __syncthreads();
  float* out = a.ATT + l * a.sATT;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = p_row(wm, mi, v, lane), dim = p_col(wn, ni, lane);
        if (row < rows) st_cg(out + (size_t)(r0 + row) * a.NA + h * HD + dim, o.c[mi][ni][v] / lrow[row]);
      }
  if (mega) signal_tile(a, in);
}
