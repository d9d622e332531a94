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
// Precision: the weights and the KV cache are bf16 values, so a product with
// them is exact once the other operand is.  Every activation operand y (fp32)
// therefore enters the matrix cores as a pair hi = bf16(y), lo = bf16(y - hi):
// y - (hi + lo) is below 2^-16 |y|, and each product is taken twice, hi W and
// lo W, into one fp32 accumulator.  Producer tiles write both parts.  A
// consumer op whose bit is clear in prefill_lo takes the hi parts only (its
// activations rounded to bf16, half the matrix-core work and activation
// traffic).
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

// prefill_lo bits: the GEMMs that take the lo parts of their activations
constexpr uint32_t P_LO_QKV = 1, P_LO_OPROJ = 2, P_LO_GATEUP = 4, P_LO_DOWN = 8;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

__device__ __forceinline__ bf16x8 as_bf16x8(v4u v) { return __builtin_bit_cast(bf16x8, v); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (lo in the low half), round to nearest even:
// one v_cvt_pk_bf16_f32 (the same result as f32_to_bf16 for finite values).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// The remainders of two floats after their packed bf16 pair `ph`, as a packed
// bf16 pair: the lo parts of the split (y - hi is exact in fp32).
__device__ __forceinline__ uint32_t pack_bf16_rest(float y0, float y1, uint32_t ph) {
  return pack_bf16(y0 - __uint_as_float(ph << 16), y1 - __uint_as_float(ph & 0xFFFF0000u));
}
// Eight floats -> (hi, lo) as two 16-byte bf16 chunks.
__device__ __forceinline__ void split8(const float* y, v4u& hi, v4u& lo) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    hi[k] = pack_bf16(y[2 * k], y[2 * k + 1]);
    lo[k] = pack_bf16_rest(y[2 * k], y[2 * k + 1], hi[k]);
  }
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
__device__ __forceinline__ void st_cg_u64(uint64_t* p, uint64_t v) {
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
  const uint16_t* xb;      // A rows (bf16 hi parts, any RMSNorm gain already applied), leading dimension K
  const uint16_t* xl;      // their lo parts, same layout
  const float* ss;         // RMSNorm: per-row sums of squares of the fp32 rows per 128-column tile
                           // [row][nss], or null (no normalisation)
  int nss;
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

// Issue the activation DMA of K step ks into LDS tile `abuf`: the hi parts
// (128 rows of 128 B, same swizzle as the weights), then the lo parts at
// abuf + PA_LO.  Rows past the tile re-read the tile's first row; their
// products are never stored.  The activation lines were written once in this
// launch by their producer tiles, with device-coherent stores, and are read
// only after those tiles' barriers (see ld_act).
constexpr int PA_LO = PBM * 128;                 // byte offset of the lo parts in an activation stage
// NP = 1 issues the hi parts only.
template <int NP>
__device__ __forceinline__ void p_issue_a(const PGemm& g, uint8_t* abuf, int ks, int wave, int lane) {
  for (int d = wave; d < PBM / 8; d += NWAVE) {
    const int row = d * 8 + lane / 8;
    const int c = (lane % 8) ^ (row & 7);
    const size_t o = (size_t)(g.r0 + (row < g.rows ? row : 0)) * g.K + ks * PKS + c * 8;
    dma_lds16<0>(g.xb + o, abuf + d * 1024);
    if constexpr (NP == 2) dma_lds16<0>(g.xl + o, abuf + PA_LO + d * 1024);
  }
}

// One K step of the tile on the matrix cores: the hi parts of the activation
// fragments against the weights, then (NP = 2) the lo parts against the same
// weights.
template <bool TWO, int NP>
__device__ __forceinline__ void p_mfma_step(const uint8_t* a, const uint8_t* b, PAcc& acc, PAcc& acc_up,
                                            int wm, int wn, int lane) {
#pragma unroll
  for (int kk = 0; kk < PKS / 16; ++kk) {
    const int chunk = kk * 2 + (lane >> 5);
    bf16x8 bfr[2], bup[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) bfr[ni] = ld_frag(b, wn * 64 + ni * 32 + (lane & 31), chunk);
    if constexpr (TWO) {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) bup[ni] = ld_frag(b, PBN + wn * 64 + ni * 32 + (lane & 31), chunk);
    }
#pragma unroll
    for (int part = 0; part < NP; ++part) {
      bf16x8 af[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) af[mi] = ld_frag(a + part * PA_LO, wm * 64 + mi * 32 + (lane & 31), chunk);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc.c[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc.c[mi][ni], 0, 0, 0);
      if constexpr (TWO) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc_up.c[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bup[ni], acc_up.c[mi][ni], 0, 0, 0);
      }
    }
  }
}

// LDS of a GEMM tile: S activation stages (hi and lo parts, 32 KB each), S
// weight stages, then the row statistics ([NT] scratch, then [PBM] row
// scales).  Three stages for one weight matrix, two for gate/up (its weight
// stages hold both matrices), so both fit one workgroup's shared memory.
constexpr int PA_STAGE = 2 * PBM * 128;
__device__ __forceinline__ constexpr int p_stages(bool two_mats) { return two_mats ? 2 : 3; }
__device__ __forceinline__ float* p_row_stats(Smem& s, bool two_mats) {
  const int st = p_stages(two_mats);
  return reinterpret_cast<float*>(s.ring + st * PA_STAGE + st * (two_mats ? 2 : 1) * PBN * 128);
}

// Full K loop of one tile.  Activations (hi and lo parts) and weights are
// DMA'd into LDS S - 1 K steps ahead of the matrix cores (S stages each);
// nothing in the loop is a register load, so the only waits are the explicit
// ones, and the loads of the next steps stay in flight while the current step
// runs.  The first weight steps are issued before the tile waits (`mega`), the
// activations after it.  Leaves the row scales (RMSNorm factors, or 1) in
// p_row_stats()[NT ..].
// TWO: gate/up (two weight matrices, acc_up accumulates the second); the
// others pass their one accumulator twice and never touch acc_up.  NP: the
// activation parts taken (2: hi and lo, 1: hi only, the activations rounded
// to bf16).
template <bool TWO, int NP>
__device__ __forceinline__ bool p_gemm(KArgs& a, Smem& s, const PGemm& g, PAcc& acc, PAcc& acc_up, bool mega,
                                       const Task in, uint32_t idx) {
  constexpr int S = TWO ? 2 : 3;                         // stages (matches p_stages)
  constexpr int D = S - 1;                               // K steps of lookahead
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  constexpr bool two = TWO;
  const int bbytes = (two ? 2 : 1) * PBN * 128;
  uint8_t* abase = s.ring;                               // S activation stages
  uint8_t* bbase = s.ring + S * PA_STAGE;                // S weight stages
  float* rs = p_row_stats(s, two);
  const int nks = g.K / PKS;

  for (int k = 0; k < D && k < nks; ++k) p_issue_b(g, bbase + k * bbytes, k, wave, lane);
  if (mega && !wait_tiles(a, in, idx)) { wait_vm<0>(); return false; }
  // row scales from the producers' sums of squares: two threads per row, each
  // summing half of the column tiles in order (loads issued eight at a time),
  // then first half + second half.  Done before the activation DMAs so the
  // wait for these loads does not also wait for them.  Unlike the activation
  // lines, one 128-byte line of partial sums has many producer tiles (one
  // float each), so an L2 may hold a copy made before all of them wrote:
  // these loads are device-coherent.
  {
    const int row = t >> 1, half = t & 1;
    float tot = 0.f;
    if (g.ss) {
      const int hn = (g.nss + 1) / 2, c0 = half * hn, c1 = min(g.nss, c0 + hn);
      const float* p = g.ss + (size_t)(g.r0 + (row < g.rows ? row : 0)) * g.nss;
      for (int c = c0; c < c1; c += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = c + j < c1 ? ld_cg(p + c + j) : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) tot += v[j];
      }
    }
    const float other = __shfl_xor(tot, 1, 64);
    const float sum = half ? other + tot : tot + other;
    if (half == 0) rs[NT + row] = g.ss ? 1.0f / sqrtf(sum / (float)g.K + a.eps) : 1.0f;
  }
  for (int k = 0; k < D && k < nks; ++k) p_issue_a<NP>(g, abase + k * PA_STAGE, k, wave, lane);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      acc.c[mi][ni] = (f32x16){};
      if constexpr (TWO) acc_up.c[mi][ni] = (f32x16){};
    }
  constexpr int NA_ = NP * PBM / 8 / NWAVE;              // activation DMAs (hi, lo) per wave per step
  // Issue order so far: the weights of steps 0 .. D-1 (before the wait), then
  // their activations.  Step 0 has landed once only the activations of steps
  // 1 .. D-1 may be outstanding; from then on each loop step issues (weights,
  // activations) of step ks + D and, after its matrix work, waits for step
  // ks + 1.
  if (D == 2 && nks > 1) wait_vm<NA_>(); else wait_vm<0>();
  __syncthreads();
  int cur = 0;                                           // stage of step ks
  for (int ks = 0; ks < nks; ++ks) {
    const bool more = ks + 1 < nks, ahead = ks + D < nks;
    const int cd = cur + D >= S ? cur + D - S : cur + D;
    if (ahead) {
      p_issue_b(g, bbase + cd * bbytes, ks + D, wave, lane);
      p_issue_a<NP>(g, abase + cd * PA_STAGE, ks + D, wave, lane);
    }
    p_mfma_step<TWO, NP>(abase + cur * PA_STAGE, bbase + cur * bbytes, acc, acc_up, wm, wn, lane);
    if (more) {
      // step ks + 1's loads have landed once only step ks + D's (if D > 1) may be outstanding
      if (D == 1 || !ahead) wait_vm<0>();
      else if (two) wait_vm<NA_ + 2 * PBN / 8 / NWAVE>();
      else wait_vm<NA_ + PBN / 8 / NWAVE>();
    }
    __syncthreads();
    cur = cur + 1 == S ? 0 : cur + 1;
  }
  if (mega) trace_mark(a, idx, 4);
  return true;
}


// Write one 128 x 128 fp32 tile staged in shared memory (ct[row][col], col
// relative to n0) as output rows: out[r][n0 + col] = ct (+ res[r][n0 + col]),
// and optionally a bf16 copy as hi and lo parts (times gain[n0 + col] when
// given) and the row's sum of squares over the tile's columns into
// ss[r][n0 / 128].  Sixteen
// threads cover one row's 128 columns, 8 consecutive columns each, so the
// stores of a wave are contiguous 512-byte runs.  Columns at or past ncols
// (a multiple of 8) and rows at or past `rows` are skipped.
struct PRowOut {
  float* out; const float* res; int ld;      // fp32 output / residual rows, leading dimension
  uint16_t* outb; uint16_t* outl;             // bf16 copy, hi and lo parts (same leading dimension), or null
  const float* gain;
  float* ss; int nss;                         // sums of squares [row][nss] or null
  int n0, ncols, r0, rows;
};

__device__ __forceinline__ void p_write_rows(const float* ct, const PRowOut& p) {
  const int t = threadIdx.x, sub = t & 15, c = sub * 8;
  constexpr int NPASS = PBM / (NT / 16);
  // every pass's residual values are loaded up front (one memory round trip
  // rather than one per pass: the stores of a pass would otherwise keep the
  // next pass's loads from being issued early)
  float4 rr[NPASS][2];
  if (p.res) {
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
      const int row = pass * (NT / 16) + (t >> 4);
      const bool valid = row < p.rows && p.n0 + c < p.ncols;
      const size_t o = (size_t)(p.r0 + (valid ? row : 0)) * p.ld + p.n0 + (valid ? c : 0);
      rr[pass][0] = ld_act4(p.res + o);
      rr[pass][1] = ld_act4(p.res + o + 4);
    }
  }
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    const int row = pass * (NT / 16) + (t >> 4);
    const bool valid = row < p.rows && p.n0 + c < p.ncols;
    float x[8];
    {
      const float4 u = *reinterpret_cast<const float4*>(ct + row * PBN + c);
      const float4 w = *reinterpret_cast<const float4*>(ct + row * PBN + c + 4);
      x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w; x[4] = w.x; x[5] = w.y; x[6] = w.z; x[7] = w.w;
    }
    float sq = 0.f;
    if (valid) {
      const size_t o = (size_t)(p.r0 + row) * p.ld + p.n0 + c;
      if (p.res) {
        const float4 u = rr[pass][0], w = rr[pass][1];
        x[0] += u.x; x[1] += u.y; x[2] += u.z; x[3] += u.w; x[4] += w.x; x[5] += w.y; x[6] += w.z; x[7] += w.w;
      }
      uint64_t* d = reinterpret_cast<uint64_t*>(p.out + o);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        st_cg_u64(d + k, (uint64_t)__float_as_uint(x[2 * k]) | ((uint64_t)__float_as_uint(x[2 * k + 1]) << 32));
#pragma unroll
      for (int k = 0; k < 8; ++k) sq += x[k] * x[k];
      if (p.outb) {
        float y[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = x[k];
        if (p.gain) {
          const float4 u = *reinterpret_cast<const float4*>(p.gain + p.n0 + c);
          const float4 w = *reinterpret_cast<const float4*>(p.gain + p.n0 + c + 4);
          y[0] *= u.x; y[1] *= u.y; y[2] *= u.z; y[3] *= u.w; y[4] *= w.x; y[5] *= w.y; y[6] *= w.z; y[7] *= w.w;
        }
        v4u hi, lo;
        split8(y, hi, lo);
        uint64_t* db = reinterpret_cast<uint64_t*>(p.outb + o);
        uint64_t* dl = reinterpret_cast<uint64_t*>(p.outl + o);
        st_cg_u64(db, (uint64_t)hi[0] | ((uint64_t)hi[1] << 32));
        st_cg_u64(db + 1, (uint64_t)hi[2] | ((uint64_t)hi[3] << 32));
        st_cg_u64(dl, (uint64_t)lo[0] | ((uint64_t)lo[1] << 32));
        st_cg_u64(dl + 1, (uint64_t)lo[2] | ((uint64_t)lo[3] << 32));
      }
    }
    if (p.ss) {
      // the 16 threads of the row, in a fixed order
      sq += __shfl_xor(sq, 8, 16);
      sq += __shfl_xor(sq, 4, 16);
      sq += __shfl_xor(sq, 2, 16);
      sq += __shfl_xor(sq, 1, 16);
      if (sub == 0 && row < p.rows) st_cg(p.ss + (size_t)(p.r0 + row) * p.nss + p.n0 / PBN, sq);
    }
  }
}

// Element (row, col) of accumulator value v of block (mi, ni) of wave (wm, wn).
__device__ __forceinline__ int p_row(int wm, int mi, int v, int lane) { return wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }
__device__ __forceinline__ int p_col(int wn, int ni, int lane) { return wn * 64 + ni * 32 + (lane & 31); }

__device__ __forceinline__ bool p_block_live(KArgs& a, int m) { return m * PBM < a.seq_len; }

// P_EMBED(m): X_0 rows of block m = embedding rows of their tokens, plus the
// bf16 copy (hi and lo parts) times the first layer's attention-norm gain and
// the rows' sums of squares per 128 columns (the QKV tiles' operands).  Each thread moves 8
// consecutive columns: one 16-byte load of bf16, four 8-byte device-coherent
// stores of fp32 and two of bf16; 16 consecutive threads cover 128 columns.
__device__ __forceinline__ void op_p_embed(KArgs& a, const Task in, uint32_t idx, bool mega) {
  const int m = in.a0;
  const uint16_t* E = static_cast<const uint16_t*>(a.embed);
  const float* gain = a.attn_norm;                        // layer 0
  const int r0 = m * PBM, rows = max(0, min(PBM, a.seq_len - r0));
  const int c8 = a.H / 8;                                 // prefill needs the hidden size a multiple of 128
  const int nss = (a.H + PBN - 1) / PBN;
  const int n = rows * c8;                                // a multiple of 16: groups of 16 threads stay together
  inject_delay(a, idx);
  constexpr int U = 4;                                    // row chunks per thread in flight at once
  for (int e0 = 0; e0 < n; e0 += NT * U) {
    v4u w[U];
    int tok[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int e = e0 + j * NT + threadIdx.x;
      const int row = e < n ? e / c8 : 0, c = e < n ? (e - row * c8) * 8 : 0;
      tok[j] = e < n ? a.tokens[r0 + row] : 0;
      const bool ok = e < n && tok[j] >= 0 && tok[j] < a.V;
      w[j] = ok ? *reinterpret_cast<const v4u*>(E + (size_t)tok[j] * a.H + c) : v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int e = e0 + j * NT + threadIdx.x;
      const bool live = e < n;
      const int row = live ? e / c8 : 0, c = live ? (e - row * c8) * 8 : 0;
      float sq = 0.f;
      if (live) {
        if ((tok[j] < 0 || tok[j] >= a.V) && c == 0)
          record_error(a, ERR_TOKEN, idx, (uint32_t)(r0 + row), (uint32_t)tok[j], (uint32_t)a.V);
        float x[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {                     // the bf16 bits are the high half of each float
          x[2 * k] = __uint_as_float(w[j][k] << 16);
          x[2 * k + 1] = __uint_as_float(w[j][k] & 0xFFFF0000u);
        }
        const size_t o = (size_t)(r0 + row) * a.H + c;
        uint64_t* dst = reinterpret_cast<uint64_t*>(a.X + o);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          st_cg_u64(dst + k, (uint64_t)__float_as_uint(x[2 * k]) | ((uint64_t)__float_as_uint(x[2 * k + 1]) << 32));
#pragma unroll
        for (int k = 0; k < 8; ++k) { sq += x[k] * x[k]; x[k] *= gain[c + k]; }
        v4u hi, lo;
        split8(x, hi, lo);
        uint64_t* db = reinterpret_cast<uint64_t*>(a.XB + o);
        uint64_t* dl = reinterpret_cast<uint64_t*>(a.XBL + o);
        st_cg_u64(db, (uint64_t)hi[0] | ((uint64_t)hi[1] << 32));
        st_cg_u64(db + 1, (uint64_t)hi[2] | ((uint64_t)hi[3] << 32));
        st_cg_u64(dl, (uint64_t)lo[0] | ((uint64_t)lo[1] << 32));
        st_cg_u64(dl + 1, (uint64_t)lo[2] | ((uint64_t)lo[3] << 32));
      }
      sq += __shfl_xor(sq, 8, 16);
      sq += __shfl_xor(sq, 4, 16);
      sq += __shfl_xor(sq, 2, 16);
      sq += __shfl_xor(sq, 1, 16);
      if (live && (threadIdx.x & 15) == 0) st_cg(a.XSS + (size_t)(r0 + row) * nss + c / PBN, sq);
    }
  }
  if (mega) signal_tile(a, in);
}

// Row stride of the QKV epilogue's staged tile: 4 floats of padding, so the
// 32 rows that the lanes of one half-wave read at the same column fall in
// different banks.
constexpr int CT_QLD = PBN + 4;

// P_QKV(m, n0, n1): one head's columns of QKV for row block m, with the
// RMSNorm row scale, QK-norm and RoPE (q, k), the KV-cache write (k, v).
__device__ __forceinline__ void op_p_qkv(KArgs& a, Smem& s, const Task in, uint32_t idx, bool mega) {
  const int l = in.layer, m = in.a0, n0 = in.a1;
  if (!p_block_live(a, m)) {
    if (mega && wait_tiles(a, in, idx)) signal_tile(a, in);
    return;
  }
  const int r0 = m * PBM, rows = min(PBM, a.seq_len - r0);
  PGemm g{a.XB + l * a.sXB, a.XBL + l * a.sXB, a.XSS + l * a.sXSS, (a.H + PBN - 1) / PBN,
          static_cast<const uint16_t*>(a.wqkv) + (size_t)l * a.NQKV * a.H, nullptr, n0, a.NQKV, a.H, r0, rows};
  PAcc acc;
  if (!((a.prefill_lo & P_LO_QKV) ? p_gemm<false, 2>(a, s, g, acc, acc, mega, in, idx)
                                  : p_gemm<false, 1>(a, s, g, acc, acc, mega, in, idx))) return;
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
        ct[row * CT_QLD + col] = acc.c[mi][ni][v] * rs[row];
      }
  __syncthreads();
  const int hh = n0 / PBN;                        // head index within [q | k | v]
  const bool is_q = hh < a.nq, is_k = !is_q && hh < a.nq + a.nkv;
  inject_delay(a, idx);
  const int row = t >> 1, part = t & 1;           // two threads per row: pairs [part*32, part*32+32)
  const int HALF = PBN / 2;
  float x0[32], x1[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) { x0[k] = ct[row * CT_QLD + part * 32 + k]; x1[k] = ct[row * CT_QLD + HALF + part * 32 + k]; }
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
    // 8-byte device-coherent stores: two floats, or four bf16 of the cache row
    float* out = a.QKV + l * a.sQKV + (size_t)pos * a.NQKV + n0;
    uint64_t* o0 = reinterpret_cast<uint64_t*>(out + part * 32);
    uint64_t* o1 = reinterpret_cast<uint64_t*>(out + HALF + part * 32);
    auto two = [](float lo, float hi) {
      return (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
    };
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      st_cg_u64(o0 + k, two(x0[2 * k], x0[2 * k + 1]));
      st_cg_u64(o1 + k, two(x1[2 * k], x1[2 * k + 1]));
    }
    if (!is_q) {
      const int gidx = hh - a.nq - (is_k ? 0 : a.nkv);
      uint16_t* cache = static_cast<uint16_t*>(is_k ? a.kc : a.vc) +
                        ((((size_t)l * a.M_cache + a.kv_row) * a.nkv + gidx) * a.ctx_max + pos) * PBN;
      uint64_t* c0 = reinterpret_cast<uint64_t*>(cache + part * 32);
      uint64_t* c1 = reinterpret_cast<uint64_t*>(cache + HALF + part * 32);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        st_cg_u64(c0 + k, (uint64_t)pack_bf16(x0[4 * k], x0[4 * k + 1]) |
                              ((uint64_t)pack_bf16(x0[4 * k + 2], x0[4 * k + 3]) << 32));
        st_cg_u64(c1 + k, (uint64_t)pack_bf16(x1[4 * k], x1[4 * k + 1]) |
                              ((uint64_t)pack_bf16(x1[4 * k + 2], x1[4 * k + 3]) << 32));
      }
    }
  }
  if (mega) signal_tile(a, in);
}

// P_OPROJ / P_DOWN: out = residual + A W^T (A = ATT_l / ACT_l; residual = X_l / HRES_l).
__device__ __forceinline__ void op_p_resid(KArgs& a, Smem& s, const Task in, uint32_t idx, bool mega, bool down) {
  const int l = in.layer, m = in.a0, n0 = in.a1;
  if (!p_block_live(a, m)) {
    if (mega && wait_tiles(a, in, idx)) signal_tile(a, in);
    return;
  }
  const int r0 = m * PBM, rows = min(PBM, a.seq_len - r0);
  const int K = down ? a.F : a.NA;
  PGemm g{down ? a.ACTB + l * a.sACTB : a.ATTB + l * a.sATTB, down ? a.ACTBL + l * a.sACTB : a.ATTBL + l * a.sATTB,
          nullptr, 0,
          static_cast<const uint16_t*>(down ? a.wdown : a.wo) + (size_t)l * a.H * K, nullptr, n0, a.H, K, r0, rows};
  PAcc acc;
  if (!((a.prefill_lo & (down ? P_LO_DOWN : P_LO_OPROJ)) ? p_gemm<false, 2>(a, s, g, acc, acc, mega, in, idx)
                                                         : p_gemm<false, 1>(a, s, g, acc, acc, mega, in, idx)))
    return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, wm = wave >> 1, wn = wave & 1;
  float* ct = reinterpret_cast<float*>(s.ring);          // [128][128] fp32 over the operand stages
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) ct[p_row(wm, mi, v, lane) * PBN + p_col(wn, ni, lane)] = acc.c[mi][ni][v];
  __syncthreads();
  // O-projection: HRES_l = X_l + ATT W_o^T, plus its bf16 copy times the FFN
  // norm gain and row sums of squares for the gate/up tiles.  Down: X_{l+1} =
  // HRES_l + ACT W_d^T, plus the same for the next layer's QKV tiles.
  const int nss = (a.H + PBN - 1) / PBN;
  const bool next = !down || l + 1 < a.L;
  PRowOut o{down ? a.X + (l + 1) * a.sX : a.HRES + l * a.sHRES, down ? a.HRES + l * a.sHRES : a.X + l * a.sX, a.H,
            next ? (down ? a.XB + (l + 1) * a.sXB : a.HB + l * a.sXB) : nullptr,
            next ? (down ? a.XBL + (l + 1) * a.sXB : a.HBL + l * a.sXB) : nullptr,
            next ? (down ? a.attn_norm + (size_t)(l + 1) * a.H : a.ffn_norm + (size_t)l * a.H) : nullptr,
            next ? (down ? a.XSS + (l + 1) * a.sXSS : a.HSS + l * a.sXSS) : nullptr, nss, n0, a.H, r0, rows};
  inject_delay(a, idx);
  p_write_rows(ct, o);
  if (mega) signal_tile(a, in);
}

// P_GATEUP: ACT = silu(RMSNorm(H) Wg^T) * (RMSNorm(H) Wu^T) for 128 columns.
__device__ __forceinline__ void op_p_gateup(KArgs& a, Smem& s, const Task in, uint32_t idx, bool mega) {
  const int l = in.layer, m = in.a0, n0 = in.a1;
  if (!p_block_live(a, m)) {
    if (mega && wait_tiles(a, in, idx)) signal_tile(a, in);
    return;
  }
  const int r0 = m * PBM, rows = min(PBM, a.seq_len - r0);
  PGemm g{a.HB + l * a.sXB, a.HBL + l * a.sXB, a.HSS + l * a.sXSS, (a.H + PBN - 1) / PBN,
          static_cast<const uint16_t*>(a.wgate) + (size_t)l * a.F * a.H,
          static_cast<const uint16_t*>(a.wup) + (size_t)l * a.F * a.H, n0, a.F, a.H, r0, rows};
  PAcc acc, up;
  if (!((a.prefill_lo & P_LO_GATEUP) ? p_gemm<true, 2>(a, s, g, acc, up, mega, in, idx)
                                     : p_gemm<true, 1>(a, s, g, acc, up, mega, in, idx))) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, wm = wave >> 1, wn = wave & 1;
  const float* rs = p_row_stats(s, true) + NT;
  float* ct = reinterpret_cast<float*>(s.ring);          // [128][128] fp32 over the operand stages
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = p_row(wm, mi, v, lane);
        const float gt = acc.c[mi][ni][v] * rs[row], u = up.c[mi][ni][v] * rs[row];
        ct[row * PBN + p_col(wn, ni, lane)] = gt / (1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * gt)) * u;
      }
  __syncthreads();
  PRowOut o{a.ACT + l * a.sACT, nullptr, a.F, a.ACTB + l * a.sACTB, a.ACTBL + l * a.sACTB, nullptr, nullptr, 0, n0,
            a.F, r0, rows};
  inject_delay(a, idx);
  p_write_rows(ct, o);
  if (mega) signal_tile(a, in);
}

// ---------------------------------------------------------------------------- causal attention tile

// P_ATTN(m, h): rows of block m attend causally to keys 0 .. last row of the
// block, read back from the KV cache (bf16) that the QKV tiles wrote.  The
// block's 128 query rows run as two halves of 64, so that Q and the
// probabilities fit shared memory as hi and lo parts.  Per half: Q
// [2 parts][2 dim halves][64 rows][128 B] (32 KB), two K blocks
// [2 dim halves][64 keys][128 B] (the next block's keys load during this one,
// 32 KB), V^T [128 dims][64 keys] (16 KB), S [64][64] fp32 (16 KB), P
// [2 parts][64][64] bf16 (16 KB) and the row statistics.  The keys and values
// are bf16 values, so S = (Q_hi + Q_lo) K^T and O = (P_hi + P_lo) V are taken
// as two products each.
constexpr int PAH = 64;                                   // query rows per half
__device__ __forceinline__ void op_p_attn(KArgs& a, Smem& s, const Task in, uint32_t idx, bool mega) {
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
  constexpr int QPART = 2 * PAH * 128;                   // one part of Q: two dim halves of 64 rows x 128 B
  uint8_t* qs = s.ring;                                  // [2 parts] x QPART
  uint8_t* ks = qs + 2 * QPART;                          // [2 dim halves][64 keys][128 B]
  uint8_t* kb1 = ks + 2 * PKB * 128;                     // the second K block
  uint8_t* vt = kb1 + 2 * PKB * 128;                     // [128 dims][64 keys] bf16, 128 B rows
  float* sm = reinterpret_cast<float*>(vt + HD * PKB * 2);   // [64][64]
  uint8_t* pb = reinterpret_cast<uint8_t*>(sm + PAH * PKB);  // [2 parts][64][64] bf16, 128 B rows
  float* mrow = reinterpret_cast<float*>(pb + 2 * PAH * PKB * 2);
  float* lrow = mrow + PAH;
  float* arow = lrow + PAH;
  float* ct = reinterpret_cast<float*>(s.ring);          // [64][128] output rows, over Q once a half is done
  // scores are kept in log2 units (scaled by log2(e) / sqrt(HD)), so every
  // exponential is one v_exp_f32; only the normalised output leaves the tile
  const float scale = 1.4426950408889634f / sqrtf((float)HD);
  // S[row][key] sits at float4 slot (key / 4) ^ (row & 15) of its row, so the
  // sixteen rows a wave's softmax reads at once hit distinct banks
  auto sidx = [](int row, int key) { return row * PKB + ((((key >> 2) ^ (row & 15)) << 2) | (key & 3)); };
  // row of accumulator value v of a 32 x 32 block of wave row wm
  auto acc_row = [&](int v) { return wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); };
  const size_t cache_rows = (((size_t)l * a.M_cache + a.kv_row) * a.nkv + g) * a.ctx_max;
  const uint16_t* Kc = static_cast<const uint16_t*>(a.kc) + cache_rows * HD;
  const uint16_t* Vc = static_cast<const uint16_t*>(a.vc) + cache_rows * HD;
  // Key blocks are double-buffered: block b + 1's keys (DMA) and values (into
  // registers, transposed into LDS at the top of block b + 1) load while block
  // b runs on the matrix cores.
  constexpr int VPT = PKB * (HD / 8) / NT;               // 16-byte value loads per thread per block
  v4u vr[VPT];
  auto load_block = [&](int k0, int nkeys, uint8_t* kdst) {
#pragma unroll
    for (int j = 0; j < VPT; ++j) {                      // values: 8 dims of one key per load, lanes on consecutive keys
      const int e = t + j * NT, key = e % PKB, d8 = (e / PKB) * 8;
      vr[j] = ld_cg_v4u(Vc + (size_t)min(k0 + key, nkeys - 1) * HD + d8);
    }
    for (int d = wave; d < 2 * PKB / 8; d += NWAVE) {     // keys: 64 x 128 dims as two 64-dim halves, 16 DMA lines
      const int half = d / (PKB / 8), key = (d % (PKB / 8)) * 8 + lane / 8;
      const int c = (lane % 8) ^ (key & 7);
      dma_lds16<1>(Kc + (size_t)min(k0 + key, nkeys - 1) * HD + half * 64 + c * 8, kdst + d * 1024);
    }
  };
  for (int hb = 0; hb * PAH < rows; ++hb) {
    const int q0 = r0 + hb * PAH;                        // first query row (position) of the half
    const int hrows = min(PAH, rows - hb * PAH);         // its valid rows
    const int nkeys = q0 + hrows;                        // causal: keys 0 .. last row of the half
    __syncthreads();                                     // the previous half's output rows are written
    // Q rows (fp32 post-RoPE) -> hi and lo bf16: four threads per row, 32 dims each
    {
      const int row = t >> 2, qtr = t & 3;
      const int dh = qtr >> 1, cb = (qtr & 1) * 4;
      const float* src = a.QKV + l * a.sQKV + (size_t)(q0 + row) * a.NQKV + h * HD + qtr * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (row < hrows) {
          const float4 u = ld_act4(src + 8 * q), w = ld_act4(src + 8 * q + 4);
          y[0] = u.x; y[1] = u.y; y[2] = u.z; y[3] = u.w; y[4] = w.x; y[5] = w.y; y[6] = w.z; y[7] = w.w;
        }
        v4u hi, lo;
        split8(y, hi, lo);
        const int off = dh * PAH * 128 + row * 128 + swz(row, cb + q) * 16;
        *reinterpret_cast<v4u*>(qs + off) = hi;
        *reinterpret_cast<v4u*>(qs + QPART + off) = lo;
      }
    }
    if (t < PAH) { mrow[t] = -INFINITY; lrow[t] = 0.f; }
    f32x16 o[2] = {(f32x16){}, (f32x16){}};              // O [64][128]: rows wm*32.., dims wn*64 + ni*32..
    load_block(0, nkeys, ks);
    for (int k0 = 0, b = 0; k0 < nkeys; k0 += PKB, ++b) {
      __syncthreads();                                   // the previous block is done with V^T and P
      // V block transposed: each thread scatters the 8 dims of its loaded keys
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int e = t + j * NT, key = e % PKB, d8 = (e / PKB) * 8;
        const uint16_t* hv = reinterpret_cast<const uint16_t*>(&vr[j]);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int dim = d8 + q;
          *reinterpret_cast<uint16_t*>(vt + dim * 128 + swz(dim, key / 8) * 16 + (key % 8) * 2) = hv[q];
        }
      }
      wait_vm<0>();                                      // this block's key DMA has landed
      if (k0 + PKB < nkeys) load_block(k0 + PKB, nkeys, (b & 1) ? ks : kb1);
      __syncthreads();
      const uint8_t* kb = (b & 1) ? kb1 : ks;
      // S = Q K^T: [64 rows][64 keys]; wave (wm, wn) computes rows wm*32.., keys wn*32..
      {
        f32x16 sc = (f32x16){};
#pragma unroll
        for (int kk = 0; kk < HD / 16; ++kk) {
          const int dh = kk / 4, chunk = (kk % 4) * 2 + (lane >> 5);
          const bf16x8 bfr = ld_frag(kb + dh * PKB * 128, wn * 32 + (lane & 31), chunk);
#pragma unroll
          for (int part = 0; part < 2; ++part)
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                ld_frag(qs + part * QPART + dh * PAH * 128, wm * 32 + (lane & 31), chunk), bfr, sc, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = acc_row(v), key = wn * 32 + (lane & 31);
          const bool ok = k0 + key <= q0 + row && k0 + key < nkeys;
          sm[sidx(row, key)] = ok ? sc[v] * scale : -INFINITY;
        }
      }
      __syncthreads();
      // online softmax per row: four threads per row, 16 keys each (four float4 reads)
      {
        const int row = t >> 2, qtr = t & 3;
        float sv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = *reinterpret_cast<const float4*>(sm + sidx(row, qtr * 16 + 4 * q));
          sv[4 * q] = v.x; sv[4 * q + 1] = v.y; sv[4 * q + 2] = v.z; sv[4 * q + 3] = v.w;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < 16; ++k) mx = fmaxf(mx, sv[k]);
        mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
        const float mold = mrow[row];
        const float mnew = fmaxf(mold, mx);
        float p[16], sum = 0.f;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          p[k] = mnew == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[k] - mnew);
          sum += p[k];
        }
        sum += __shfl_xor(sum, 1, 64);
        sum += __shfl_xor(sum, 2, 64);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          v4u hi, lo;
          split8(p + 8 * c, hi, lo);
          const int off = row * 128 + swz(row, qtr * 2 + c) * 16;
          *reinterpret_cast<v4u*>(pb + off) = hi;
          *reinterpret_cast<v4u*>(pb + PAH * 128 + off) = lo;
        }
        __syncthreads();
        if (qtr == 0) {
          const float al = mold == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mold - mnew);
          arow[row] = al;
          lrow[row] = lrow[row] * al + sum;
          mrow[row] = mnew;
        }
      }
      __syncthreads();
      // O = O * alpha + P V: A = P [64 rows][64 keys] (hi, lo), B = V^T [128 dims][64 keys]
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float al = arow[acc_row(v)];
        o[0][v] *= al;
        o[1][v] *= al;
      }
#pragma unroll
      for (int kk = 0; kk < PKB / 16; ++kk) {
        const int chunk = kk * 2 + (lane >> 5);
        bf16x8 bfr[2];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) bfr[ni] = ld_frag(vt, wn * 64 + ni * 32 + (lane & 31), chunk);
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const bf16x8 af = ld_frag(pb + part * PAH * 128, wm * 32 + (lane & 31), chunk);
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) o[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr[ni], o[ni], 0, 0, 0);
        }
      }
    }
    __syncthreads();
    // ATT_l rows of head h for this half, and their bf16 copy (hi, lo) for the O-projection tiles
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = acc_row(v);
        ct[row * PBN + wn * 64 + ni * 32 + (lane & 31)] = o[ni][v] / lrow[row];
      }
    __syncthreads();
    PRowOut po{a.ATT + l * a.sATT, nullptr, a.NA, a.ATTB + l * a.sATTB, a.ATTBL + l * a.sATTB, nullptr, nullptr, 0,
               h * HD, a.NA, q0, hrows};
    if (hb == 0) inject_delay(a, idx);
    p_write_rows(ct, po);
  }
  if (mega) signal_tile(a, in);
}
