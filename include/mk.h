/*
 * mk.h -- C ABI of the tile-synchronized decoder megakernel for MI355X (gfx950).
 *
 * One decode step (or one prefill) of a pre-norm Llama/Qwen decoder runs as a
 * single persistent kernel.  Every workgroup is an interpreter that pops
 * instructions from a queue in device memory; each instruction computes one
 * tile of one intermediate tensor and first waits on barrier counters of
 * exactly the producer tiles it reads.  The LM head runs as a separate kernel.
 * The same op bodies also run one kernel per operator, for comparison.
 *
 * Sources of the method (the pages this library implements; each entry point
 * below names the passage it follows):
 *  - MegaOps abstract: dependencies enforced on individual tiles of the
 *    intermediate tensor a producer writes and a consumer reads, instead of
 *    whole-kernel barriers; weight prefetch while the producer still runs.
 *  - "Production Megakernels" lecture summary, Key takeaways: one work queue
 *    built with symbolic sequence (S) and context (P) lengths; barriers are
 *    tensors partitioned by dependency.  Technical details: an on-device
 *    interpreter (a loop around a switch) whose cores atomically pop
 *    instructions from a global queue in DRAM; memory pipelining across tiles.
 *    Practical implications: the LM head kept outside the megakernel; the host
 *    kept out of the hot loop.
 *
 * Conventions for every entry point:
 *  - Returns MK_OK (0) or a negative mk_status.  On error nothing is enqueued
 *    (every check, including the kernels' shared-memory and residency limits,
 *    runs before the first launch) and mk_last_error() holds a message
 *    (thread-local).
 *  - Pointers named d_* and the fields of mk_weights / mk_kv are device
 *    pointers; everything else is host memory.
 *  - The caller owns and allocates all device memory (weights, KV cache,
 *    workspace, device queue copy, outputs).  The library allocates only the
 *    host mk_queue object (and, in MK_KERNEL_PER_OP_GRAPH mode, the HIP
 *    runtime's graph objects) and never calls hipMalloc; it never
 *    synchronises, except mk_device_error, which synchronises the given
 *    stream, and the eviction of a cached graph (see MK_KERNEL_PER_OP_GRAPH).
 *  - Launches go to the caller's stream and return asynchronously.
 *  - Host-side state (options, kernel attributes, the graph cache) is guarded
 *    by one process-wide lock, so the entry points may be called from several
 *    threads.  On the device: kernel-per-op calls (eager or graph) with
 *    distinct workspaces may run concurrently on different streams.  A
 *    megakernel call (decode or prefill) needs every one of its workgroups
 *    resident at once, and two megakernels in flight on one device can hold
 *    the compute units the other needs: megakernel calls must be serialised
 *    per device (one stream, or ordered streams).  Calls that share a
 *    workspace race.
 *  - Matrices use the [out, in] row-major layout; all layers of one kind are
 *    stacked contiguously ([n_layers][out][in]).
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mk_status;
enum {
  MK_OK = 0,
  MK_EINVAL = -1,    /* bad argument, shape or tile plan */
  MK_ENOMEM = -2,    /* host allocation failed */
  MK_ELAUNCH = -3,   /* a HIP launch or runtime call failed */
  MK_EDEVICE = -4,   /* the device reported an error (mk_device_error) */
  MK_ENOTSUP = -5    /* valid request this build does not implement */
};

enum { MK_F32 = 0, MK_BF16 = 1 };                     /* element type of matrices and KV cache */
enum { MK_DECODE = 0, MK_PREFILL = 1 };               /* queue mode */
/* Execution modes: the persistent interpreter; the same op bodies one kernel
 * per (layer, op) segment in stream order; those per-op launches captured
 * into a HIP graph and replayed (decode only); and one kernel per segment on
 * several streams, synchronised on tiles (decode only). */
enum { MK_MEGAKERNEL = 0, MK_KERNEL_PER_OP = 1, MK_KERNEL_PER_OP_GRAPH = 2, MK_MULTI_STREAM = 3 };
enum { MK_PART_META = 0, MK_PART_INSTR = 1, MK_PART_WAITS = 2, MK_PART_TARGETS = 3,
       MK_PART_DEVICE = 4 };

/* Decoder shape.  Norm gains are always fp32.  rope_theta: base of the rotary
 * frequencies theta^(-2i/head_dim), pairs (i, i + head_dim/2). */
typedef struct mk_config {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  int32_t qk_norm;        /* per-head RMSNorm of q and k before RoPE (Qwen3) */
  int32_t has_embed;      /* 0: input rows are given as fp32 (d_x0) */
  int32_t has_lm_head;    /* 0: no final norm / LM head / argmax */
  int32_t dtype;          /* MK_F32 or MK_BF16 */
  float rms_eps;
  double rope_theta;
} mk_config;

/* Tile plan: explicit, never inferred.  tq/to/tf/td are the output-column tile
 * widths of the QKV, O-projection, gate/up and down GEMVs; kb keys per
 * attention split (decode); bm x bn the prefill GEMM tile (bn holds whole
 * heads).  rows: B for decode (1..32), S_max for prefill.  n_queues: workers
 * pop from n_queues sub-queues; instruction i belongs to sub-queue i mod
 * n_queues (1..1024; with as many sub-queues as workers the assignment of
 * instructions to workers is static). */
typedef struct mk_plan {
  int32_t mode, rows, ctx_max;
  int32_t tq, to, tf, td, kb, bm, bn;
  int32_t n_queues;
  int32_t fuse_combine;   /* decode: 0 = split-combine instructions (COMBINE).
                           * 1 = none; each O-projection tile waits on the
                           * attention split partials and merges them while
                           * staging (bit 0 of the META word after bn).
                           * 2 = none; every split counts its arrival on its
                           * (row, KV head) partial tile, whose target is
                           * then NS + 1: the split that arrives last merges
                           * the partials into the attention output and
                           * signals the tile once more, and the O-projection
                           * tiles wait on those tiles and read the merged
                           * rows (bit 2 of that word).  All three give the
                           * same results bit for bit. */
  int32_t loop;           /* decode: 1 = a queue for mk_decode_loop (persistent
                           * multi-step decode): each step ends with LM-head
                           * tiles of 64 vocabulary rows (LMHEAD) and one argmax
                           * per row (ARGMAX), and the next step's embedding
                           * tiles wait on the previous step's argmax (flagged
                           * waits); needs an embedding and an LM head (0 or 1;
                           * recorded in bit 1 of the META word after bn) */
  int32_t attn_pop;       /* decode, single-step queues: 1 = in the megakernel, a
                           * layer's attention splits are handed out at run time
                           * ("Production Megakernels" lecture summary, Technical
                           * details: cores pop work atomically, so faster ones
                           * pick up the slack).  The first worker to reach one
                           * of its split positions in a layer takes splits in
                           * queue order from a per-layer counter until none are
                           * left, then skips its other split positions of that
                           * layer.  Each split still waits on and signals its own
                           * tiles, so results equal the static order's bit for
                           * bit; with ragged contexts the workers' loads even
                           * out.  Needs one sub-queue per worker (else the order
                           * stays static); the other modes keep one split per
                           * workgroup.  0 or 1; bit 3 of the META word after bn;
                           * not with loop. */
} mk_plan;

typedef struct mk_queue mk_queue;   /* opaque, host memory */

/* Build the instruction queue and its tile barriers for (cfg, plan).
 * Follows the lecture summary's Key takeaways (a single work queue built once
 * with the sequence and context lengths symbolic; barriers are tensors
 * partitioned by dependency) and the MegaOps abstract (each dependency is on
 * the tiles of the intermediate tensor a consumer reads).
 * Host only, deterministic: equal inputs give byte-identical parts.
 * Layout of the parts (little-endian):
 *   META    u32 magic 'TMK1', version 1, mode, n_instr, n_barriers,
 *           n_wait_ranges, n_segments, n_queues, rows, ctx_max, n_splits,
 *           n_layers, tq, to, tf, td, kb, bm, bn, flags (bit 0: split
 *           combines fused into the O-projection; bit 1: loop queue; bit 2:
 *           split combines merged by the last split), then n_segments x
 *           {op, layer, first, count} (maximal runs of one op of one layer)
 *   INSTR   n_instr x 32 B {u16 op, u16 layer, u32 a0, a1, a2, wait_off,
 *           wait_cnt, signal, n_wait}
 *   WAITS   n_wait_ranges x {u32 first barrier, u32 count}; bit 31 of count
 *           marks barriers of the previous step (loop queues: at step t a
 *           same-step barrier is complete at target * (t + 1) signals, a
 *           previous-step one at target * t)
 *   TARGETS n_barriers x u32 (instructions that signal each barrier, plus
 *           one for a partial tile whose last split merges: flags bit 2)
 *   DEVICE  INSTR | WAITS | TARGETS, each starting on a 256-byte boundary:
 *           what mk_decode_step / mk_prefill read from d_queue.
 * Ownership: *out is a host object the caller releases with mk_queue_free.
 * Errors: MK_EINVAL for a bad shape or plan, MK_ENOMEM. */
mk_status mk_build_queue(const mk_config* cfg, const mk_plan* plan, mk_queue** out);
/* Bytes of one part (0 for an unknown part or a NULL queue). */
size_t mk_queue_nbytes(const mk_queue* q, int32_t part);
/* Copy one part into host_dst, which holds exactly mk_queue_nbytes(q, part)
 * bytes (MK_EINVAL otherwise).  The caller uploads the DEVICE part into device
 * memory it owns (the lecture summary's queue in DRAM). */
mk_status mk_queue_export(const mk_queue* q, int32_t part, void* host_dst, size_t nbytes);
/* Release a queue (NULL is ignored), with any HIP graphs captured for it. */
void mk_queue_free(mk_queue* q);

/* Device workspace: per-layer intermediate tensors, split partials, barrier
 * counters (the lecture summary's barriers as tensors; the MegaOps abstract's
 * per-tile dependencies), queue heads, error record; for a prefill queue also
 * the bf16 copies of the GEMM activation operands and per-row sums of squares
 * that the producer tiles write for their consumers.  No alignment beyond 256
 * bytes needed.
 * mk_workspace_offset gives the byte offset of one tensor (MK_T_*) of one
 * layer inside it (layer 0..n_layers for MK_T_X; 0 for the others that are not
 * per layer). Intermediates are fp32 row-major [rows][cols].
 * Errors: MK_EINVAL (NULL arguments, unknown tensor, layer out of range). */
enum { MK_T_X = 0, MK_T_QKV = 1, MK_T_OPART = 2, MK_T_ATT = 3, MK_T_HRES = 4, MK_T_ACT = 5,
       MK_T_COUNTERS = 6, MK_T_HEADS = 7, MK_T_ERROR = 8, MK_T_LMPART = 9 };
mk_status mk_workspace_nbytes(const mk_queue* q, size_t* nbytes);
mk_status mk_workspace_offset(const mk_queue* q, int32_t tensor, int32_t layer, size_t* offset);

typedef struct mk_weights {
  const void* wqkv;        /* [L][(nq + 2 nkv) hd][H]; rows: q heads, k heads, v heads */
  const void* wo;          /* [L][H][nq hd] */
  const void* wgate;       /* [L][F][H] */
  const void* wup;         /* [L][F][H] */
  const void* wdown;       /* [L][H][F] */
  const float* attn_norm;  /* [L][H] */
  const float* ffn_norm;   /* [L][H] */
  const float* q_norm;     /* [L][hd]  (qk_norm only) */
  const float* k_norm;     /* [L][hd]  (qk_norm only) */
  const void* embed;       /* [V][H]   (has_embed only) */
  const void* lm_head;     /* [V][H]   (has_lm_head only) */
  const float* final_norm; /* [H]      (has_lm_head only) */
} mk_weights;

/* KV cache: [L][rows][n_kv][ctx_max][hd] in the model dtype, keys after RoPE.
 * rows: sequences the cache holds (decode: 0 or the batch; prefill: >= 1). */
typedef struct mk_kv {
  void* k;
  void* v;
  int32_t rows;
} mk_kv;

/* One decode step for `batch` sequences (must equal the queue's rows).
 * Follows the lecture summary's Technical details (the persistent
 * interpreter: every workgroup pops instructions from the queue in device
 * memory, runs one tile each; memory pipelining across tiles) and the MegaOps
 * abstract (a consumer tile starts once the producer tiles it reads are done,
 * streaming its weights while it waits).
 * Row b's new token sits at position d_ctx_lens[b] (< ctx_max): its key and
 * value are written there and attention covers positions 0..d_ctx_lens[b].
 * The caller advances d_ctx_lens between steps (the library keeps no state
 * between steps).  Inputs: d_tokens [batch] token ids (has_embed), else d_x0
 * [batch][H] fp32 rows.  Outputs: d_logits [batch][V] fp32 and d_next [batch]
 * (argmax, lowest index on ties); either may be NULL to skip; both ignored
 * without an LM head.  The final hidden rows are the workspace tensor MK_T_X
 * of layer n_layers.
 * exec_mode MK_MEGAKERNEL: counter reset, one persistent interpreter launch,
 * LM head, argmax.  MK_KERNEL_PER_OP: error-record reset, the same op bodies,
 * one launch per (layer, op), stream-ordered, no tile waits (the whole-kernel
 * barriers the MegaOps abstract measures against).  MK_KERNEL_PER_OP_GRAPH:
 * the per-op launches of the first call with a given set of arguments
 * (pointers, queue, options) are captured into a HIP graph that this and later
 * calls with the same arguments replay; the kernels read tokens, context
 * lengths and inputs from device memory, so a replay sees their current
 * values.  At most 16 graphs are cached (least recently used evicted, after
 * waiting for its last replay); mk_queue_free drops a queue's graphs.
 * MK_MULTI_STREAM (the MegaOps abstract's multi-stream form: dependent kernels
 * overlap and synchronise on tiles of the intermediate tensor, no fusion):
 * counter reset, then one kernel per (layer, op) segment, the segments dealt
 * round-robin to MK_OPT_STREAMS internal streams (default priority, created on
 * a device's first such call and kept until the process ends), each
 * instruction waiting on and signalling the megakernel's tile counters; the
 * caller's stream waits for all of them before the LM head.  Each kernel gets
 * 8 * floor(workers_per_cu * (CUs / 8) / streams) workgroups, which stride
 * over its instructions, so the at most `streams` kernels active at once
 * are resident together and every wait ends.  Like the megakernel, a
 * multi-stream call needs those compute units: serialise it with other
 * megakernel or multi-stream calls on the device.  All four modes give
 * bitwise equal results.
 * Errors: MK_EINVAL (mismatched queue / sizes / null pointers), MK_ENOTSUP
 * (tiles that do not fit a workgroup's shared memory; megakernel workgroups
 * that cannot all be resident), MK_ELAUNCH.  A loop queue is refused (it runs
 * through mk_decode_loop). */
mk_status mk_decode_step(const mk_queue* q, const void* d_queue, const mk_weights* w,
                         const mk_kv* kv, const int32_t* d_tokens, const float* d_x0,
                         const int32_t* d_ctx_lens, int32_t batch, void* d_workspace,
                         size_t workspace_nbytes, float* d_logits, int32_t* d_next,
                         int32_t exec_mode, hipStream_t stream);

/* Persistent multi-step decode: `steps` decode steps of a loop queue
 * (mk_plan.loop = 1) in one launch.  Follows the lecture summary's Practical
 * implications (the host stays out of the hot loop; the forward pass
 * re-executes on the device): the interpreter runs the queue `steps` times,
 * each step's LM-head tiles and per-row argmax inside the megakernel, and the
 * next step's embedding tiles wait (tile-granular) on the previous step's
 * argmax.  Counters are cleared once, before the launch.
 * Step t of row b sits at position d_ctx_lens[b] + t (the caller's d_ctx_lens
 * is not changed; a position outside the cache is a device error).
 * feedback 0 (teacher-forced): d_tokens is [steps][batch], step t embeds
 * d_tokens[t]; feedback 1 (greedy): d_tokens is [batch], step 0 embeds it and
 * step t > 0 embeds the argmax of step t - 1.  d_next [steps][batch] (required)
 * receives every step's argmax (lowest index on ties); d_logits [steps][batch][V]
 * fp32 (nullable) every step's logits.  The final hidden rows of the last step
 * are the workspace tensor MK_T_X of layer n_layers.  bf16 models only.
 * Errors: MK_EINVAL (not a loop queue, sizes, null pointers), MK_ENOTSUP
 * (fp32 model; workgroups that cannot all be resident), MK_ELAUNCH. */
mk_status mk_decode_loop(const mk_queue* q, const void* d_queue, const mk_weights* w, const mk_kv* kv,
                         const int32_t* d_tokens, const int32_t* d_ctx_lens, int32_t batch, int32_t steps,
                         int32_t feedback, void* d_workspace, size_t workspace_nbytes, float* d_logits,
                         int32_t* d_next, hipStream_t stream);

/* mk_decode_step without a workspace argument, for callers that cannot
 * allocate device memory or pass one (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  The step's workspace is a
 * static device array of MK_STATIC_SCRATCH_BYTES (64 MiB) inside the library,
 * one per device, held until the process ends; no hipMalloc, hipFree or
 * allocating library routine is called.  A queue whose workspace
 * (mk_workspace_nbytes) exceeds it is refused with MK_EINVAL.  exec_mode:
 * MK_MEGAKERNEL or MK_KERNEL_PER_OP (graph and multi-stream modes allocate
 * runtime objects: MK_EINVAL).  The
 * other arguments and the results are those of mk_decode_step.  d_error
 * (nullable, device, 8 x u32) receives the step's device error record
 * (mk_dev_error, then 3 zero words) when the step ends, since the scratch
 * holding it is not the caller's.  Every call on a device shares that
 * device's scratch and leaves its contents there (counters and the error
 * record are cleared at the start of each call): calls that overlap on one
 * device race, whatever their streams. */
#define MK_STATIC_SCRATCH_BYTES (64u << 20)
mk_status mk_decode_step_static(const mk_queue* q, const void* d_queue, const mk_weights* w,
                                const mk_kv* kv, const int32_t* d_tokens, const float* d_x0,
                                const int32_t* d_ctx_lens, int32_t batch, float* d_logits,
                                int32_t* d_next, uint32_t* d_error, int32_t exec_mode,
                                hipStream_t stream);

/* The LM head on its own (the second half of mk_decode_step): final RMSNorm
 * of the workspace's last hidden rows (MK_T_X of layer n_layers, written by a
 * previous mk_decode_step on the same stream and workspace), the vocabulary
 * GEMV into d_logits [rows][V] fp32, and the argmax into d_next [rows] (lowest
 * index on ties); either output may be NULL.  Follows the lecture summary's
 * Practical implications: the LM head stays outside the megakernel (mixed
 * execution); calling it separately lets a caller time the two parts.
 * Errors: MK_EINVAL (no LM head, not a decode queue, sizes), MK_ELAUNCH. */
mk_status mk_lm_head(const mk_queue* q, const mk_weights* w, void* d_workspace, size_t workspace_nbytes,
                     float* d_logits, int32_t* d_next, hipStream_t stream);

/* Causal prefill of seq_len (1 .. the queue's rows) tokens of one sequence into
 * cache row kv_row (< kv->rows), positions 0..seq_len-1.  Follows the lecture
 * summary's Key takeaways (the queue is built once for S_max with the sequence
 * length symbolic: row blocks at or past seq_len are no-ops that still signal)
 * and Technical details (the same interpreter over the prefill queue; an
 * attention tile of row block m waits only on the key / value tiles of row
 * blocks <= m).  d_logits_last [V] and d_next [1] receive the last position's
 * logits and argmax (the LM head as a separate kernel, Practical
 * implications).  The GEMM tiles run on the matrix cores with bf16 operands
 * (each producer tile also writes its output rounded to bf16, times the
 * consuming RMSNorm's gain where there is one) and fp32 accumulation.
 * Requires a bf16 model with an embedding, hidden size a multiple of 128, the
 * FFN and attention widths multiples of 64, head_dim 128 and 128 x 128 tiles
 * (MK_ENOTSUP otherwise).  exec_mode: MK_MEGAKERNEL or MK_KERNEL_PER_OP.  The
 * per-layer hidden rows are the workspace tensors, [S_max][...] fp32.
 * Errors: MK_EINVAL, MK_ENOTSUP, MK_ELAUNCH. */
mk_status mk_prefill(const mk_queue* q, const void* d_queue, const mk_weights* w,
                     const mk_kv* kv, const int32_t* d_tokens, int32_t seq_len, int32_t kv_row,
                     void* d_workspace, size_t workspace_nbytes, float* d_logits_last,
                     int32_t* d_next, int32_t exec_mode, hipStream_t stream);

/* Device-side error record, written by a worker whose bounded wait on a
 * barrier expired (the kernel then drains instead of hanging), or by an op
 * that met an input outside its range.  Not from the pages: the library's own
 * watchdog.  Every call clears it before its first kernel runs. */
typedef struct mk_dev_error {
  uint32_t code;       /* 0 none; 1 barrier wait timed out; 2 unknown opcode;
                          3 context length outside the cache; 4 token id outside the vocabulary */
  uint32_t instr;      /* instruction index */
  uint32_t barrier;    /* barrier id */
  uint32_t value;      /* counter value seen */
  uint32_t target;     /* target it waited for */
} mk_dev_error;
/* Synchronises `stream`, then copies the record out.  Returns MK_EDEVICE when
 * the record holds an error, MK_OK otherwise. */
mk_status mk_device_error(const mk_queue* q, const void* d_workspace, mk_dev_error* out,
                          hipStream_t stream);

/* Tuning knobs (process-wide; not from the pages): */
enum {
  MK_OPT_WORKERS_PER_CU = 0,  /* megakernel workgroups per compute unit (default 1); a
                               * launch whose workgroups the registers or shared memory
                               * cannot all hold at once is refused with MK_ENOTSUP
                               * (a worker waits on tiles of others, so all must run) */
  MK_OPT_SPIN_LIMIT = 1,      /* polls before a barrier wait gives up (default 1<<22) */
  MK_OPT_NUM_CUS = 2,         /* read-only: compute units of the current device */
  /* Trace mode: a device buffer (value = its address) of at least 64 bytes per
   * instruction.  While set, each megakernel instruction i writes 8 x u64 at
   * offset 64*i: (workgroup << 32 | XCD id), pop time, time its waits ended,
   * phase A (inputs staged), phase B (main loop done), end time, the time
   * an attention split that arrived last began its merge (fuse_combine 2), 0
   * (device wall clock, 100 MHz; a phase an op does not have stays 0).  Set the
   * address to 0 to stop. */
  MK_OPT_TRACE_BUFFER = 3,
  MK_OPT_TRACE_BYTES = 4,
  /* How decode GEMVs issue their weight lines: 0 (default) and 1 keep the
   * ring's lines in flight while staged inputs are read, 2 lets the compiler
   * order them (it waits for every line in flight before each read of the
   * staged inputs).  Results are identical. */
  MK_OPT_GEMV_PIPE = 5,
  /* Race check: a non-zero 32-bit seed makes every tile's producer stall for a
   * pseudo-random time drawn from (seed, instruction index), 0 to about 50 us,
   * before it stores the tile.  A consumer that read a tile without waiting
   * for its barrier would then read the workspace's previous contents.
   * Results are identical to a run without it; 0 (default) turns it off. */
  MK_OPT_DELAY_SEED = 6,
  /* Internal streams of MK_MULTI_STREAM, 1..8 (default 2). */
  MK_OPT_STREAMS = 7,
  /* MK_MEGAKERNEL: megakernel launches per decode step, 1..8 (default 1).  With
   * K > 1 the step is a composition of K megakernels ("One Megakernel is Not
   * Enough" abstract: cutting the model into several megakernels), cut at layer
   * boundaries: launch k runs the instructions of layers [k L / K, (k + 1) L / K),
   * the first also the embedding, in stream order, so tiles of earlier
   * launches are complete before a later one starts; results are identical bit
   * for bit.  Needs a single-step queue with one sub-queue per worker and at
   * most L launches (else MK_ENOTSUP).  An error recorded by one launch stops
   * it; each worker of a later launch of the step then spends at most one
   * barrier spin limit before it stops too, and mk_device_error reports the
   * first error. */
  MK_OPT_MEGAKERNELS = 8,
  /* mk_prefill: which GEMMs take both bf16 parts (hi, lo) of their fp32
   * activations, a bit mask (1 QKV, 2 O-projection, 4 gate/up, 8 down; default
   * 15, all).  A GEMM whose bit is clear takes the hi parts only: its
   * activations are rounded to bf16 and it runs half the matrix-core products. */
  MK_OPT_PREFILL_LO = 9
};
/* Errors: MK_EINVAL for an unknown or read-only key or a value out of range. */
mk_status mk_set_option(int32_t key, int64_t value);
/* The option's value, or -1 for an unknown key. */
int64_t mk_get_option(int32_t key);

/* Static name of a status, and the calling thread's last error message. */
const char* mk_status_str(mk_status s);
const char* mk_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
