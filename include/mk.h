/* mk.h -- C ABI of the MI355X persistent decode megakernel (one GPU).
 *
 * One autoregressive decode step of a Llama-style decoder -- embedding
 * lookup, RMSNorm, QKV projection + RoPE + KV-cache append, GQA attention over
 * the bf16 KV cache, O-projection + residual, RMSNorm, SwiGLU MLP + residual,
 * final RMSNorm, LM head and greedy argmax -- runs as ONE launched kernel that
 * executes a fine-grained task graph.
 *
 * Sources of the method (web pages, cited by title and section):
 *  - "Compilar LLM en un MegaKernel para lograr inferencia de baja latencia"
 *    (GeekNews summary of the Mirage Persistent Kernel post), sections
 *    "Parte 1. Compilador" (operator graph -> fine-grained task graph of tasks
 *    and events) and "Parte 2. Runtime" (workers, schedulers, event counters
 *    with thresholds, 1-2 us inter-task overhead).
 *  - "MPK: A Compiler and Runtime for Mega-Kernelizing Tensor Programs"
 *    (gist.science explainer), sections 2-4 (tGraph, in-kernel runtime with
 *    ahead-of-time vs just-in-time task launch, paged shared memory).
 *  - "Llama-70B向け低レイテンシ・高スループットMegakernelの公開" (hakusoku.com
 *    summary of the Hazy Research post), section 命令セットの再設計 (fused
 *    RMS norm, QKV matmul + RoPE, attention, O-proj + residual instructions;
 *    matrix-vector bodies for latency, matrix-matrix for throughput).
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

#define MK_ABI_VERSION 1

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

/* How a step is executed.  Both modes run the same task bodies. */
enum {
  MK_MODE_MEGAKERNEL = 0, /* one persistent cooperative launch per step (currently
                             refused; see mk_create) */
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
  MK_FLAG_SPIN_LIMIT_1 = 1u << 5, /* test hook: every in-kernel wait gives up after one unsuccessful
                                     check, so a step ends in MK_ERR_TIMEOUT without any wave hanging */
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
 * KV cache bf16.  Shapes must satisfy: hidden, ffn and n_q_heads*head_dim are
 * multiples of 8; head_dim is 64 or 128; n_q_heads is a multiple of
 * n_kv_heads. */
typedef struct {
  int32_t abi_version; /* must be MK_ABI_VERSION */
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  float rms_eps;       /* RMSNorm epsilon (added to mean(x^2) inside the root) */
  float rope_theta;    /* RoPE base */
  int32_t tie_embeddings; /* nonzero: the LM head is the embedding table */
  int32_t max_batch;   /* sequences decoded together (1..64) */
  int32_t max_seq;     /* KV-cache capacity in positions */
  int32_t mode;        /* MK_MODE_* */
  uint32_t flags;      /* MK_FLAG_* */
  uint32_t watchdog_ms;/* in-kernel dependency wait limit; 0 = 2000 ms */
  int32_t num_cus;     /* persistent grid size; 0 = every CU of the device */
  int32_t attn_split;  /* positions per split-KV attention task; 0 = automatic (64) */
  int32_t kv_fp32;     /* KV cache element type: 0 = bf16, nonzero = fp32 */
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

/* Create a decoder on the current HIP device.  Validates the config, builds
 * and validates the task graph on the host, allocates the KV cache, activation
 * scratch, event counters and task tables (handle-owned), and uploads the
 * tables.  `hip_stream` is a hipStream_t (NULL = default stream); every later
 * call is ordered on it.  Synchronous w.r.t. the host.
 * MK_MODE_MEGAKERNEL returns MK_ERR_UNSUPPORTED: its cooperative launch never
 * completed on the gfx950 test device, and it stays off until the cause is found. */
mk_status mk_create(const mk_config* cfg, const mk_weights* weights, void* hip_stream, mk_handle** out);

/* Prefill: runs positions 0..P-1 of B sequences (d_tokens int32 [B, P],
 * row-major) through the decode graph one position at a time, and writes the
 * greedy token of the last position to d_next int32 [B].  If d_logits is not
 * NULL, the last position's logits are written to it (fp32 [B, vocab]).
 * Requires length == 0; sets the batch size B (1..max_batch) and length = P.
 * P + length must not exceed max_seq (MK_ERR_CAPACITY). */
mk_status mk_prefill(mk_handle* h, const int32_t* d_tokens, int32_t B, int32_t P,
                     int32_t* d_next, float* d_logits);

/* One decode step for every sequence: token ids d_in int32 [B] at position
 * `length`; writes greedy ids to d_out int32 [B] (lowest index among equal
 * maxima) and, if d_logits is not NULL, the logits fp32 [B, vocab].  d_out may
 * be the d_in of the next call (no host round trip).  length += 1.
 * MK_ERR_CAPACITY if length == max_seq (nothing enqueued). */
mk_status mk_decode_step(mk_handle* h, const int32_t* d_in, int32_t* d_out, float* d_logits);

/* Wait for the stream; returns MK_ERR_TIMEOUT (and poisons the handle) if an
 * in-kernel watchdog fired during any earlier step. */
mk_status mk_synchronize(mk_handle* h);

/* length := 0 and batch unset; KV contents become undefined.  Clears a
 * poisoned state only for MK_ERR_STATE caused by misuse, not by a timeout. */
mk_status mk_reset(mk_handle* h);

/* Describe the KV cache (device pointers owned by the handle). */
mk_status mk_kv_view(mk_handle* h, mk_kv_layout* out);

/* Copy the whole K and V caches (layout of mk_kv_view, every allocated
 * position) into host memory: `bytes` must equal one cache's size,
 * n_layers * max_batch * n_kv_heads * max_seq * head_dim * elem_bytes.
 * Waits for the stream first; synchronous.  For checking a long cache
 * against the oracle, which then continues from the imported state. */
mk_status mk_kv_read(mk_handle* h, void* k_host, void* v_host, int64_t bytes);

/* Message of the last failed mk_* call on this thread ("" if none). */
const char* mk_last_error(void);

/* Free everything the handle owns (waits for its stream first).  NULL-safe. */
void mk_destroy(mk_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
