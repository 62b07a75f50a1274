/* mk_debug.h -- inspection and single-body entry points of libmk (tests,
 * profiling).  Same conventions as mk.h: device pointers are HIP device
 * memory, errors are reported through mk_status + mk_last_error().
 */
#ifndef MK_DEBUG_H
#define MK_DEBUG_H

#include "mk.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ---- task graph (host only; no GPU needed) ------------------------------
 * The graph cuts every operator of one decode step into wavefront-sized tasks
 * placed on per-CU queues and wired by counting events ("Compilar LLM en un
 * MegaKernel ...", section "Parte 1. Compilador"). */
typedef struct {
  int32_t n_tasks, n_events, n_stages, ncu, nsplit, split;
  int32_t max_queue, min_queue;        /* tasks per CU */
  int64_t max_cu_bytes, min_cu_bytes;  /* weight bytes streamed per CU per step */
  int64_t weight_bytes;                /* all weight bytes of one step */
} mk_graph_info;

/* Build the graph for `cfg` on `ncu` CUs and run the static validator
 * (coverage, topological queues, thresholds, read-after-write covered by
 * waits, RoPE pairs whole).  MK_ERR_INVALID_ARG with the validator's message
 * on failure.  For max_batch >= 2 the graph is the batched launch plan: one
 * stage per launch (n_stages), each stage's tasks its workgroups (max_queue /
 * min_queue: the largest and smallest stage), validated for coverage of
 * every projection's (row group, K chunk) pairs, of every output element and
 * split partial, and for reads of earlier stages only; n_events, the per-CU
 * byte fields are 0 and weight_bytes is what the projections stream. */
mk_status mk_graph_inspect(const mk_config* cfg, int32_t ncu, mk_graph_info* out);

/* Test hook for the batched graph's validator (max_batch >= 2): build the
 * graph, plant one mistake, validate.  fault: 1 a projection workgroup takes
 * the row block of its neighbour, 2 a finishing task takes its neighbour's
 * row group, 3 the O projection's launch moves before the attention merge, 4
 * the down projection's finishing launch expects one K split more than ran,
 * 5 the last attention split of a KV head repeats the first.  Returns
 * MK_ERR_INVALID_ARG with the validator's message when it catches the mistake,
 * MK_OK when it does not, MK_ERR_UNSUPPORTED if the config has no place for
 * that mistake (e.g. no split projection). */
mk_status mk_batched_graph_fault(const mk_config* cfg, int32_t ncu, int32_t fault);

typedef struct {
  int32_t completed;     /* 1 if every task ran */
  int32_t executed;      /* tasks run before completion or deadlock */
  int32_t blocked_event; /* on deadlock: an event a blocked task waits on, else -1 */
  int32_t race;          /* 1 if a task or staging read incomplete data */
} mk_sim_result;

/* Execute the graph's queues on the CPU under the runtime protocol in a random
 * interleaving (seeded).  drop_event >= 0 suppresses one signal of that event
 * (fault injection). `workers` = worker waves per CU (1..kWaves-1). */
mk_status mk_graph_simulate(const mk_config* cfg, int32_t ncu, uint64_t seed, int32_t workers, int32_t drop_event,
                            mk_sim_result* out);

/* Copy the graph's tasks in global order into `out` (48 bytes per task,
 * layout of the internal Task struct) and the CU of each task into `cu`.
 * Either may be NULL; `cap` is the capacity in tasks. Returns the count in *n. */
mk_status mk_graph_export(const mk_config* cfg, int32_t ncu, void* out, int32_t* cu, int32_t cap, int32_t* n);

/* ---- internal buffers of a handle (device pointers, fp32) ------------------ */
typedef struct {
  float* xs;        /* [L+1][B][H]: xs[l+1] = residual stream after layer l */
  float* xmid;      /* [L][B][H]:   residual after attention of layer l */
  float* q;         /* [L][B][nq*hd]: rotated queries */
  float* attn_out;  /* [L][B][nq*hd]: attention output before O-proj */
  float* h;         /* [L][B][F]: SwiGLU output */
  uint32_t* events; /* event counters */
  int32_t n_events, n_tasks, ncu, nsplit, split;
  int32_t lds_bytes; /* dynamic LDS of the persistent kernel */
  uint32_t exact_ops; /* per-operator mode: bit t set when operator type t runs
                         the variant without row/column clamps (its rows fill
                         whole tiles and its columns whole prefetch rounds) */
  int32_t op_grid[9];  /* per-operator mode: workgroups of each GEMV operator's
                          last launch (index = task type) */
} mk_debug_view;
mk_status mk_get_debug_view(mk_handle* h, mk_debug_view* out);

/* Kernel status words (synchronous): [0] abort flag, [1] error code (0 ok,
 * 1 timeout, 2 non-finite logits, 3 token id out of range), then for a
 * megakernel timeout: [2] workgroup, [3] wave (0..3 stagers, 4..7 compute
 * waves), [4] (operator index << 8) | wait kind (1 input page, 2 compute
 * completions, 3 stager rendezvous, 4 tagged operator input, 5 queries/keys/
 * values, 6 attention records, 7 LM-head keys), [5] value seen or progress,
 * [6] value needed, [7] 3. */
mk_status mk_read_status(mk_handle* h, uint32_t out[16]);

/* Timestamps of the per-operator path's wave timelines (see mk_trace_op),
 * when created with MK_FLAG_TRACE: *n = entry pairs, in ticks of the device
 * wall clock (`ticks_per_us` returned).  Synchronous. */
mk_status mk_read_trace(mk_handle* h, uint64_t* out, int32_t cap, int32_t* n, double* ticks_per_us);

/* Megakernel timestamps of the last step (MK_MODE_MEGAKERNEL created with
 * MK_FLAG_TRACE), in ticks of the device wall clock (*ticks_per_us).  Layout
 * out[(k * ncu + w) * slots + j] for GEMV operator k (k = 4 l + {0 QKV, 1 O,
 * 2 gate/up, 3 down}; k = 4 L the LM head), workgroup w, with C = slots - 10
 * compute waves:
 *   j < C     compute wave j: (duration << 32) | (end mod 2^32), from the
 *             moment it saw the input page published to the end of its
 *             epilogues;
 *   j = C     the moment the workgroup's first stager published its part of
 *             the page (64-bit);
 *   j = C + 1 the stager started polling operator k's input words;
 *   j = C + 2 every word of the input had arrived;
 *   j = C + 3 .. C + 9 (k = 4 l + 1 only, 0 elsewhere): an attention unit of
 *             this workgroup had its query/key/value words (C + 3), had
 *             written its record (C + 4); a merge of this workgroup had its
 *             wave-0 share of the records (C + 5), had written its output
 *             (C + 6); the unit's waves had met after staging the queries
 *             (C + 7), its wave 0 had stored its softmax state (C + 8), the
 *             waves had met after storing theirs (C + 9) (the last such unit
 *             or merge of the workgroup).
 * *ops, *ncu and *slots give the dimensions; with out NULL only those are
 * returned.  cap = capacity of out in words.  Synchronous. */
mk_status mk_mega_trace(mk_handle* h, uint64_t* out, int64_t cap, int32_t* ops, int32_t* ncu, int32_t* slots,
                        double* ticks_per_us);

/* The megakernel's hand-over buffers (device pointers; 64-bit words, fp32
 * value bits in the low half and the epoch of the step that wrote them in
 * the high half): x [L+1][H] (row l+1 = residual after layer l), xmid [L][H],
 * qkv [L][(nq + 2 nkv) hd] (rotated q, rotated k, v of the last position),
 * attn [L][nq hd], h [L][F]; epoch = the epoch of the last enqueued step. */
typedef struct {
  const uint64_t *x, *xmid, *qkv, *attn, *h;
  uint32_t epoch;
} mk_mega_view;
mk_status mk_get_mega_view(mk_handle* h, mk_mega_view* out);

/* HBM streaming-read probe: reads `bytes` (a multiple of 16) of src with
 * 16-byte non-temporal loads from `wgs` workgroups of 512 threads, `loads`
 * loads in flight per thread (4, 8 or 16), `reps` times on `stream`;
 * *best_ms = the fastest repetition (HIP events).  Synchronous. */
mk_status mk_t_stream_read(const void* src, int64_t bytes, int32_t wgs, int32_t loads, int32_t reps, void* stream,
                           float* best_ms);

/* Per-operator wave timeline (MK_MODE_PER_OP, batch 1, handle created with
 * MK_FLAG_TRACE | MK_FLAG_NO_GRAPH): from now on the waves of operator
 * `type` of `layer` log four wall-clock stamps each into the trace buffer
 * read by mk_read_trace: entry 4*w (w = block * waves per block + wave) =
 * (XCC_ID << 60 | HW_ID bits 0..27 << 32) | start (low 32 bits), then three
 * stamps.  GEMV operators (1 QKV, 4 O, 5 GU, 6 DOWN, 7 LM; 8 waves per
 * block): input staged, weight stream done, epilogues done.  Attention (2;
 * 4 waves per block, 8 for the single-split kernel): queries staged,
 * positions done, records written.  type < 0 stops logging. */
mk_status mk_trace_op(mk_handle* h, int32_t type, int32_t layer);

/* Time operators with HIP events on the handle's stream (MK_MODE_PER_OP):
 * every launch of a task type whose bit (1 << type, types 1..8 = QKV, ATTN,
 * MERGE, O, GU, DOWN, LM, ARGMAX; type 0 = the RMSNorm launches of the batched
 * path) is set in type_mask is bracketed by an event
 * pair, up to max_launches launches.  mk_read_op_times waits for the stream,
 * returns per-type total milliseconds and launch counts in arrays of 9
 * (index = type), and stops timing. */
mk_status mk_time_ops(mk_handle* h, uint32_t type_mask, int32_t max_launches);
mk_status mk_read_op_times(mk_handle* h, double* total_ms, int32_t* launches);

/* Back-to-back replay (MK_MODE_PER_OP, after at least one prefill): enqueues
 * only the launches of operator `type` (0 = the RMSNorm launches of the
 * batched path, 1 QKV, 2 ATTN, 3 MERGE, 4 O, 5 GU, 6 DOWN) of one decode step,
 * for every layer, `reps` times in a row on the handle's stream between two
 * HIP events, with the arguments of the last step.  Cycling through all
 * layers keeps the weights from being served out of the last-level cache.
 * The sequence state is unchanged: batch 1 stages each launch's input from
 * per-layer buffers, so a replay rewrites the same outputs from the same
 * inputs; the batched path shares its operand planes across layers, so its
 * replays read the last-written planes (same shapes and bytes) and write only
 * buffers that the next step rewrites before reading -- which is why its QKV
 * launches (they append to the KV cache) are refused.  The LM head and argmax
 * are refused on both paths (their argmax state carries into the next step).
 * Waits for the stream; *total_ms = elapsed time, *launches = kernels
 * launched. */
mk_status mk_time_op_replay(mk_handle* h, int32_t type, int32_t reps, double* total_ms, int32_t* launches);

/* The shipped single-sequence GEMV operator kernel of `type` (1 QKV, 4 O,
 * 5 gate/up, 6 down, 7 LM head) for `layer` (0 for the LM head), in the
 * launch configuration a decode step uses (grid, task split, EXACT or
 * clamped instance), on explicit buffers: the input x (fp32 device, K = hidden
 * for QKV, gate/up and the LM head, n_q_heads * head_dim for O, ffn for down)
 * is staged as it is, without RMSNorm, and the operator's raw dot products go
 * to y (fp32 device) at their rows of the operator's matrix -- QKV:
 * [Wq; Wk; Wv] ((n_q + 2 n_kv) head_dim rows), gate/up: [Wgate; Wup]
 * (2 ffn rows), the others their own row count -- instead of the epilogues
 * (no RoPE, cache append, residual, SwiGLU or argmax; the handle's sequence
 * state is untouched).  Asynchronous on the handle's stream.  max_batch 1
 * handles only (MK_ERR_UNSUPPORTED otherwise). */
mk_status mk_t_op_raw(mk_handle* h, int32_t type, int32_t layer, const float* x, float* y);

/* Rows (sequence x position) per chunk of the batched prefill of a handle
 * created with MK_FLAG_BATCHED_PREFILL: rows in [max_batch, 4096]; a chunk
 * then holds rows / max_batch positions of every sequence (the tests use
 * small chunks to cross chunk boundaries).  MK_ERR_STATE without the flag,
 * MK_ERR_INVALID_ARG outside the range. */
mk_status mk_t_set_prefill_rows(mk_handle* h, int32_t rows);

/* ---- single task bodies on explicit buffers (asynchronous on `stream`) ----- */
/* y[N] = W[N,K] x[K]; W bf16 row-major, x/y fp32; K a multiple of 8. */
mk_status mk_t_gemv(const void* W, const float* x, float* y, int32_t N, int32_t K, void* stream);
/* y = x * (mean(x^2) + eps)^-1/2 * gamma; gamma bf16; n a multiple of 8. */
mk_status mk_t_rmsnorm(const float* x, const void* gamma, float eps, float* y, int32_t n, void* stream);
/* Decode attention of one sequence: q fp32 [nq, hd]; k, v (bf16, or fp32 if
 * kv_f32) with head g at k + g*head_stride elements, position p at + p*hd; T
 * positions; split-KV partials of `split` positions merged by log-sum-exp;
 * o fp32 [nq, hd].  Synchronous (allocates and frees its partial buffer). */
mk_status mk_t_attention(const float* q, const void* k, const void* v, int64_t head_stride, int32_t nq, int32_t nkv,
                         int32_t hd, int32_t T, int32_t split, int32_t kv_f32, float* o, void* stream);
/* mk_t_attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and result, but the split records live in a static
 * per-device array of 2^20 floats (4 MiB), held by each GPU the library runs
 * on until the process ends, and the call is asynchronous on `stream` (no
 * allocation, no free, no synchronization).  Needs nkv * ceil(T / split) *
 * (nq / nkv) * (hd + 2) <= 2^20 (MK_ERR_CAPACITY otherwise; use a larger
 * split).  All calls on one GPU share its array: calls that overlap in time on
 * one GPU (other streams, other threads) race and must be serialised by the
 * caller.  Arguments and other errors as mk_t_attention. */
mk_status mk_t_attention_noalloc(const float* q, const void* k, const void* v, int64_t head_stride, int32_t nq,
                                 int32_t nkv, int32_t hd, int32_t T, int32_t split, int32_t kv_f32, float* o,
                                 void* stream);
/* Batched projection body (matrix cores): Y[b][n] = sum_k W[n][k] *
 * (A[0][b][k] + A[1][b][k]) for b < B, n < N; W bf16 [N, K]; A bf16
 * [2][Bp][K], the hi and lo planes of the activations, with Bp = 16, 32 or 64
 * rows (the smallest that holds B; rows B..Bp-1 of both planes must be zero);
 * Y fp32 [B, N]; K a multiple of 8, 1 <= B <= 64.  tiled != 0: W is in the
 * layout of mk_tile_weights (N a multiple of 16, K of 32). */
mk_status mk_t_bgemm(const void* W, const void* A, float* Y, int32_t N, int32_t K, int32_t B, int32_t tiled,
                     void* stream);
/* out[0] = lowest index of the maximum of x[n] (fp32).  Synchronous. */
mk_status mk_t_argmax(const float* x, int32_t n, int32_t* out, void* stream);

/* Device facts used by the runtime: compute units, wall-clock ticks per us,
 * max dynamic LDS per workgroup. */
mk_status mk_device_info(int32_t* ncu, double* ticks_per_us, int32_t* max_lds);

#ifdef __cplusplus
}
#endif
#endif /* MK_DEBUG_H */
