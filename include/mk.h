/* mk.h -- C ABI of the MI355X persistent decode megakernel (one GPU).
 *
 * One autoregressive decode step of a Llama-style decoder -- embedding
 * lookup, RMSNorm, QKV projection + RoPE + KV-cache append, GQA attention over
 * the KV cache, O-projection + residual, RMSNorm, SwiGLU MLP + residual,
 * final RMSNorm, LM head and greedy argmax -- split into fine-grained tasks.
 *
 * How a step runs (mk_config.mode):
 *  - MK_MODE_MEGAKERNEL (one sequence): ONE ordinary kernel launch per step.
 *    Every compute unit holds one persistent workgroup of eight waves: four
 *    stager waves stage each operator's input into LDS (with the RMSNorm
 *    gain), run the split-KV attention units and the log-sum-exp merges;
 *    four compute waves pull the operator's GEMV tasks from an LDS task pool
 *    and run the fused epilogues (RoPE + KV append, residuals, SwiGLU, LM-head
 *    argmax).  Dependencies between workgroups travel as epoch-tagged data
 *    words: a consumer re-reads a word until it carries the step's epoch.
 *  - MK_MODE_PER_OP: the same task bodies as one kernel launch per operator,
 *    replayed as one captured HIP graph per step (the comparison build).
 *  - max_batch >= 2 always runs per operator, with matrix-core (MFMA) bodies.
 * The KV cache is bf16 or fp32 (mk_config.kv_fp32), in either mode.
 *
 * Sources of the method (web pages, cited by title and section):
 *  - "Compilar LLM en un MegaKernel para lograr inferencia de baja latencia"
 *    (GeekNews summary of the Mirage Persistent Kernel post), sections
 *    "Parte 1. Compilador" (operator graph -> fine-grained task graph of tasks
 *    and events) and "Parte 2. Runtime" (workers, schedulers, event-driven
 *    execution inside one kernel, 1-2 us inter-task overhead).
 *  - "MPK: A Compiler and Runtime for Mega-Kernelizing Tensor Programs"
 *    (gist.science explainer), sections 1 and 3 (one kernel for the whole
 *    program; an in-kernel runtime that starts tasks when their inputs are
 *    ready).
 *  - hakusoku summary of the Hazy Research megakernel posts,
 *    "全てのGPUを購入したので、徹底的にそのGPUを活用します。", section
 *    高スループットMegakernelの設計と工夫 / 命令セットの再設計 (fused RMS norm, QKV
 *    matmul + RoPE, attention, O-proj + residual instructions; matrix-vector
 *    bodies for latency, matrix-matrix for throughput).
 *  - "Cómo la fusión de kernels CUDA acelera la inferencia de LLM", section
 *    "Sigue los datos intermedios" (residual + norm fusion, SwiGLU FFN fusion).
 *
 * Conventions for every function below:
 *  - All device pointers are HIP device memory on the handle's device.
 *  - Calls are asynchronous on the handle's stream unless stated otherwise;
 *    host-side validation errors return immediately and enqueue nothing.
 *  - On error the message is available from mk_last_error() (thread-local,
 *    valid until the next mk_* call on the same thread).
 *  - A handle is not thread-safe; separate handles are independent.
 */
#ifndef MK_H
#define MK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_ABI_VERSION 2

typedef struct mk_handle mk_handle; /* opaque */

typedef enum {
  MK_OK = 0,
  MK_ERR_INVALID_ARG = -1,   /* bad pointer, size or config field */
  MK_ERR_OUT_OF_MEMORY = -2, /* a device allocation failed */
  MK_ERR_HIP = -3,           /* a HIP runtime call failed (message has the HIP error) */
  MK_ERR_CAPACITY = -4,      /* KV cache full (length == max_seq) or batch > max_batch */
  MK_ERR_TIMEOUT = -5,       /* in-kernel watchdog fired: a dependency never arrived */
  MK_ERR_STATE = -6,         /* call not valid in the current state, or handle poisoned */
  MK_ERR_UNSUPPORTED = -7    /* valid request this build does not implement */
} mk_status;

/* How a step is executed (see the top of this file). */
enum {
  MK_MODE_MEGAKERNEL = 0, /* one persistent launch per step (max_batch 1) */
  MK_MODE_PER_OP = 1      /* one kernel launch per operator, the same task bodies */
};

/* Flags (mk_config.flags). */
enum {
  MK_FLAG_TRACE = 1u << 0,  /* record per-task {cu, task, start, end} timestamps */
  MK_FLAG_POISON = 1u << 1,  /* fill activation scratch with NaN before every step */
  MK_FLAG_NO_GRAPH = 1u << 2, /* per-op mode: launch every operator eagerly instead of
                                 replaying the step as one captured HIP graph */
  MK_FLAG_FUSED_MERGE = 1u << 3, /* per-op mode: run the attention log-sum-exp merge in the last
                                    split workgroup of each KV group instead of as its own launch */
  MK_FLAG_SPIN_LIMIT_1 = 1u << 5, /* megakernel test hook: every in-kernel wait gives up after one
                                     unsuccessful check, so a step ends in MK_ERR_TIMEOUT with every
                                     wave exiting normally */
  MK_FLAG_BATCHED_PREFILL = 1u << 6, /* mk_prefill runs every prompt position at once, in chunks of
                                        4096 rows (sequence x position): the projections as bf16
                                        matrix-core GEMMs on split fp32 activations, causal attention
                                        over the cache; either mode.  Needs row-major weights.  Without
                                        it, prefill runs one decode step per position */
  MK_FLAG_SHUFFLE = 1u << 7, /* megakernel mode: deal every GEMV operator's tasks to the
                                workgroups in a rotated order, the rotation drawn per operator and
                                step from mk_config.debug_seed.  Which workgroup runs a task, and
                                when, must not change any result: the test suite compares the
                                outputs bit for bit with and without it (a race or an
                                order-dependent result would show as a difference).  A shuffled
                                handle runs the generic megakernel instance (clamped loads), whose
                                arithmetic is the same.  Per-operator and batched handles refuse
                                it (MK_ERR_INVALID_ARG) */
  MK_FLAG_TILED_WEIGHTS = 1u << 4 /* batched path (max_batch >= 2): wq, wk, wv, wo, w_gate, w_up,
                                     w_down and (untied) lm_head are stored in the tiled layout that
                                     mk_tile_weights writes; embed and the norm gains stay
                                     row-major.  Needs every projection's row count a multiple of
                                     16 and its column count a multiple of 32 (mk_create checks). */
};

/* Converts a row-major bf16 matrix W [N][K] (device memory) into the tiled
 * layout of MK_FLAG_TILED_WEIGHTS, in dst (device, N*K elements, distinct
 * from src), asynchronously on `hip_stream` (NULL: the default stream).
 * Layout: 16 x 32 blocks; block (i, j) starts at element (i * K/32 + j) * 512
 * and holds, at element 8*l + e (l < 64, e < 8), W[16i + l mod 16][32j +
 * 8*floor(l/16) + e] -- the 16 bytes lane l supplies to one 16x16x32
 * matrix-core step, so a wave reads each block as one contiguous kilobyte.
 * Errors: MK_ERR_INVALID_ARG for NULL or equal pointers, N not a multiple of
 * 16 or K not a multiple of 32. */
mk_status mk_tile_weights(const void* src, void* dst, int64_t N, int64_t K, void* hip_stream);

/* Model shape and runtime options.  Weights are bf16, activations fp32, the
 * KV cache bf16 or fp32 (kv_fp32).  Shapes must satisfy: hidden, ffn and
 * n_q_heads*head_dim are multiples of 8; head_dim is 64 or 128; n_q_heads is
 * a multiple of n_kv_heads.  MK_MODE_MEGAKERNEL further needs max_batch 1,
 * 1, 2, 4 or 8 query heads per KV head, vocab <= 131072, n_q_heads <= 256 and
 * at most 256 compute units (num_cus). */
typedef struct {
  int32_t abi_version; /* must be MK_ABI_VERSION */
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  float rms_eps;       /* RMSNorm epsilon (added to mean(x^2) inside the root) */
  float rope_theta;    /* RoPE base */
  int32_t tie_embeddings; /* nonzero: the LM head is the embedding table */
  int32_t max_batch;   /* sequences decoded together (1..64); every prefill
                          must use exactly this many (see mk_prefill) */
  int32_t max_seq;     /* KV-cache capacity in positions */
  int32_t mode;        /* MK_MODE_* */
  uint32_t flags;      /* MK_FLAG_* */
  uint32_t watchdog_ms;/* in-kernel dependency wait limit; 0 = 2000 ms */
  int32_t num_cus;     /* workgroups per operator (megakernel: persistent grid size);
                          0 = every CU of the device */
  int32_t attn_split;  /* positions per split-KV attention task; 0 = automatic (64) */
  int32_t kv_fp32;     /* KV cache element type: 0 = bf16, nonzero = fp32 */
  uint32_t debug_seed; /* seed of MK_FLAG_SHUFFLE's task orders; ignored without it */
} mk_config;

/* Weights: bf16 bit patterns, row-major [out, in], contiguous, device memory.
 * Owned by the caller and must outlive the handle; never written. */
typedef struct {
  const void* embed;      /* [vocab, hidden] */
  const void* lm_head;    /* [vocab, hidden]; NULL iff tie_embeddings */
  const void* final_norm; /* [hidden] */
  /* host arrays of n_layers device pointers each */
  const void* const* attn_norm; /* [hidden] */
  const void* const* wq;        /* [n_q_heads*head_dim, hidden] */
  const void* const* wk;        /* [n_kv_heads*head_dim, hidden] */
  const void* const* wv;        /* [n_kv_heads*head_dim, hidden] */
  const void* const* wo;        /* [hidden, n_q_heads*head_dim] */
  const void* const* ffn_norm;  /* [hidden] */
  const void* const* w_gate;    /* [ffn, hidden] */
  const void* const* w_up;      /* [ffn, hidden] */
  const void* const* w_down;    /* [hidden, ffn] */
} mk_weights;

/* Layout of the handle-owned KV cache (element strides; elements are bf16 or
 * fp32, see elem_bytes):
 * K[l][b][g][p][d] at k + l*stride_layer + b*stride_batch + g*stride_head + p*stride_pos + d. */
typedef struct {
  void* k;
  void* v;
  int64_t stride_layer, stride_batch, stride_head, stride_pos;
  int32_t length;     /* positions currently valid */
  int32_t batch;      /* sequences in use (0 before the first prefill) */
  int32_t elem_bytes; /* 2 (bf16) or 4 (fp32) */
} mk_kv_layout;

/* Create a decoder on the current HIP device ("Compilar LLM en un MegaKernel
 * ...", section "Parte 1. Compilador": the operator graph is split into tasks
 * and their dependencies before anything runs).  Validates the config, builds
 * and validates the task graph on the host, allocates the KV cache, the
 * activation and hand-over buffers and the task tables (handle-owned), and
 * uploads the tables.  `hip_stream` is a hipStream_t (NULL = default stream);
 * every later call is ordered on it.  Synchronous w.r.t. the host.
 * Errors: MK_ERR_INVALID_ARG for a bad config or weight table,
 * MK_ERR_UNSUPPORTED for a shape or mode combination this build does not run
 * (the message names it), MK_ERR_OUT_OF_MEMORY, MK_ERR_HIP. */
mk_status mk_create(const mk_config* cfg, const mk_weights* weights, void* hip_stream, mk_handle** out);

/* Prefill: runs positions 0..P-1 of B sequences (d_tokens int32 [B, P],
 * row-major) through the decode graph one position at a time, and writes the
 * greedy token of the last position to d_next int32 [B].  If d_logits is not
 * NULL, the last position's logits are written to it (fp32 [B, vocab]).  The
 * pages' workload feeds a prompt before generating ("Compilar LLM en un
 * MegaKernel ...", section "Valor central de MPK": a 39-token prompt, then
 * 512 generated tokens); filling the cache with the decode step itself is
 * this library's reading.  Requires length == 0; sets length = P.  B must
 * equal max_batch: a handle is built for one batch size (task split, MFMA
 * tiles, cache layout), so a smaller batch uses a handle created for it
 * (B outside [1, max_batch]: MK_ERR_CAPACITY; 1 <= B < max_batch:
 * MK_ERR_UNSUPPORTED).  P must not exceed max_seq (MK_ERR_CAPACITY).  In
 * MK_MODE_MEGAKERNEL the P positions run in one launch.  With
 * MK_FLAG_BATCHED_PREFILL (either mode) every position of every sequence
 * runs at once instead, in chunks of 4096 rows: the projections as bf16
 * matrix-core GEMMs on fp32 activations split into a high and a low bf16
 * part, causal attention over the cache, the same KV cache and outputs (to
 * fp32 rounding; prefill as the throughput counterpart of decode: "Cómo la
 * fusión de kernels CUDA acelera la inferencia de LLM", section "Comprueba si
 * la fusión ha ayudado").  Asynchronous on the handle's stream in every case;
 * a GEMM library error returns MK_ERR_HIP. */
mk_status mk_prefill(mk_handle* h, const int32_t* d_tokens, int32_t B, int32_t P,
                     int32_t* d_next, float* d_logits);

/* One decode step for every sequence ("Compilar LLM en un MegaKernel ...",
 * section "Parte 2. Runtime": the whole step's task graph executes inside one
 * kernel in megakernel mode): token ids d_in int32 [B] at position `length`;
 * writes greedy ids to d_out int32 [B] (lowest index among equal maxima) and,
 * if d_logits is not NULL, the logits fp32 [B, vocab].  d_out may be the d_in
 * of the next call (no host round trip).  length += 1.
 * Without a prefill the first step runs at position 0 for max_batch
 * sequences.  MK_ERR_CAPACITY if length == max_seq, MK_ERR_STATE on a
 * poisoned handle (nothing enqueued in either case). */
mk_status mk_decode_step(mk_handle* h, const int32_t* d_in, int32_t* d_out, float* d_logits);

/* n_steps greedy decode steps of one sequence (max_batch 1) from token id
 * d_in[0] at position `length`: step i's greedy id goes to d_out[i] (int32
 * [n_steps], device) and is the input of step i + 1; if d_logits is not NULL
 * the last step's logits go there (fp32 [vocab]).  In MK_MODE_MEGAKERNEL the
 * n_steps steps run in ONE launch ("Compilar LLM en un MegaKernel ...",
 * section "Panorama general y ventajas": the whole inference in a single
 * kernel, no launch per step): the argmax of step i reaches every workgroup
 * as a tagged word that step i + 1's embedding lookup waits for.  Per
 * operator, each step is one graph launch with the id fed back on the
 * device.  length += n_steps.  MK_ERR_CAPACITY if length + n_steps >
 * max_seq, MK_ERR_UNSUPPORTED for max_batch > 1 (nothing enqueued). */
mk_status mk_generate(mk_handle* h, const int32_t* d_in, int32_t n_steps, int32_t* d_out, float* d_logits);

/* Wait for the stream; returns MK_ERR_TIMEOUT (and poisons the handle) if an
 * in-kernel watchdog fired during any earlier step.  In megakernel mode a host
 * watchdog also raises an abort word that every in-kernel wait polls, if the
 * stream has not drained within 10 s plus 100 ms per step enqueued since the
 * last wait, so that every wave exits.  (No passage defines this call: the
 * pages' runtime has no host interface.) */
mk_status mk_synchronize(mk_handle* h);

/* length := 0 and batch unset; KV contents become undefined.  Clears a
 * poisoned state only for MK_ERR_STATE caused by misuse, not by a timeout.
 * (Host plumbing; no passage.) */
mk_status mk_reset(mk_handle* h);

/* Describe the KV cache (device pointers owned by the handle; the pages fix
 * no cache layout, this is the library's). */
mk_status mk_kv_view(mk_handle* h, mk_kv_layout* out);

/* Copy the whole K and V caches (layout of mk_kv_view, every allocated
 * position) into host memory: `bytes` must equal one cache's size,
 * n_layers * max_batch * n_kv_heads * max_seq * head_dim * elem_bytes.
 * Waits for the stream first; synchronous.  For checking a long cache
 * against the oracle, which then continues from the imported state. */
mk_status mk_kv_read(mk_handle* h, void* k_host, void* v_host, int64_t bytes);

/* Message of the last failed mk_* call on this thread ("" if none).  (Host
 * plumbing; no passage.) */
const char* mk_last_error(void);

/* Free everything the handle owns (waits for its stream first).  NULL-safe.
 * (Host plumbing; no passage.) */
void mk_destroy(mk_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
