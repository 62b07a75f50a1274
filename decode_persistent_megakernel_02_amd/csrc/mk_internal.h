// Internal structures shared by the host task-graph builder and the device
// runtime.  Not part of the public ABI.
//
// The task graph follows the MPK description ("Compilar LLM en un MegaKernel
// ...", section "Parte 1. Compilador"): each operator is cut into tasks that
// each run on one compute unit, and tasks are wired through events; a task
// signals its output event when done, and an event is "fired" once its counter
// reaches a threshold (section "Parte 2. Runtime", event-driven execution).
#pragma once
#include <stdint.h>

namespace mk {

constexpr int kWave = 64;
constexpr int kWaves = 8;             // waves per workgroup (1 scheduler + workers)
constexpr int kWorkers = kWaves - 1;  // worker waves per CU in the persistent kernel
constexpr int kMaxGqa = 8;            // query heads per KV head supported
constexpr int kMaxSplit = 4096;       // positions per split-KV attention task
#ifndef MK_ATTN_WAVES
#define MK_ATTN_WAVES 4
#endif
constexpr int kAttnWaves = MK_ATTN_WAVES;         // waves per split in the per-operator attention kernel
#ifndef MK_OP_WGS_PER_CU
#define MK_OP_WGS_PER_CU 1
#endif
constexpr int kOpWgsPerCu = MK_OP_WGS_PER_CU;  // per-operator GEMV grid: workgroups per CU (1 measured best)
#ifndef MK_XCDS
#define MK_XCDS 8
#endif
constexpr int kXcds = MK_XCDS;        // accelerator complex dies (each with its own L2) of the device
constexpr int kAttnFullWaves = 8;     // waves of the whole-context attention kernel
constexpr int kLocalSlots = 64;       // per-CU LDS counters for aggregated event signals
constexpr int kMaxBatch = 64;         // sequences per step
constexpr int kPrefillRows = 4096;    // batched prefill: rows (sequence x position) per chunk
constexpr int kMaxTasksPerWave = 64; // GEMV results a wave of a per-operator kernel holds in LDS (<= wave size:
                                      // lane j runs the epilogue of task j)
constexpr int kBgemmWaves = 4;        // waves per workgroup of the batched (MFMA) projections
constexpr int kNormThreads = 256;     // threads per row of the batched RMSNorm kernel
constexpr uint16_t kNone16 = 0xFFFF;
constexpr uint8_t kNone8 = 0xFF;

// Task types.
enum TaskType : uint8_t {
  TT_QKV = 1,     // rows of Wq/Wk/Wv on norm(x); epilogue RoPE, q -> scratch, k/v -> cache
  TT_ATTN = 2,    // split-KV partial (m, l, o) for one (batch row, KV group, split)
  TT_MERGE = 3,   // log-sum-exp merge of the splits of one (batch row, KV group)
  TT_O = 4,       // rows of Wo on attention output; epilogue residual add
  TT_GU = 5,      // rows of W_gate and W_up on norm(xmid); epilogue SwiGLU
  TT_DOWN = 6,    // rows of W_down on h; epilogue residual add
  TT_LM = 7,      // rows of the LM head on norm(x_L); epilogue logits + argmax partial
  TT_ARGMAX = 8   // reduce the argmax partials -> next token
};

// Staged-input kinds (what the LDS activation page holds).
enum StageKind : uint16_t {
  SK_NONE = 0,
  SK_ATTN_NORM = 1,  // rmsnorm(x_l) * gamma_attn[l]   (x_0 = embedding row)
  SK_O_IN = 2,       // attention output of layer l
  SK_FFN_NORM = 3,   // rmsnorm(xmid_l) * gamma_ffn[l]
  SK_H = 4,          // SwiGLU output of layer l
  SK_FINAL_NORM = 5  // rmsnorm(x_L) * gamma_final
};
inline constexpr uint16_t stage_key(int kind, int layer) { return (uint16_t)((kind << 12) | (layer + 1)); }
inline constexpr int stage_kind(uint16_t key) { return key >> 12; }
inline constexpr int stage_layer(uint16_t key) { return (key & 0xFFF) - 1; }

// Shape of a GEMV task per operator: R weight rows streamed together, D
// 512-column chunks of each row in flight (R * D * 16 B per lane, 16 KiB per
// wave).  The per-operator kernels double-buffer tasks, so a wave holds up to
// two such buffers.  Long rows (down-projection, K = ffn) take one row.
// The defaults can be overridden at build time (MK_SHAPE_<OP>_R / _D) to tune
// for another device; the host graph builder and the kernels read the same
// values.
#ifndef MK_SHAPE_QKV_R
#define MK_SHAPE_QKV_R 2
#endif
#ifndef MK_SHAPE_QKV_D
#define MK_SHAPE_QKV_D 4
#endif
#ifndef MK_SHAPE_O_R
#define MK_SHAPE_O_R 2
#endif
#ifndef MK_SHAPE_O_D
#define MK_SHAPE_O_D 4
#endif
#ifndef MK_SHAPE_GU_R
#define MK_SHAPE_GU_R 2
#endif
#ifndef MK_SHAPE_GU_D
#define MK_SHAPE_GU_D 4
#endif
#ifndef MK_SHAPE_DOWN_R
#define MK_SHAPE_DOWN_R 2
#endif
#ifndef MK_SHAPE_DOWN_D
#define MK_SHAPE_DOWN_D 4
#endif
#ifndef MK_SHAPE_LM_R
#define MK_SHAPE_LM_R 2
#endif
#ifndef MK_SHAPE_LM_D
#define MK_SHAPE_LM_D 4
#endif
template <int TT> struct TaskShape;
template <> struct TaskShape<1> { static constexpr int R = MK_SHAPE_QKV_R, D = MK_SHAPE_QKV_D; };    // QKV: one RoPE pair or R v rows
template <> struct TaskShape<4> { static constexpr int R = MK_SHAPE_O_R, D = MK_SHAPE_O_D; };        // O
template <> struct TaskShape<5> { static constexpr int R = MK_SHAPE_GU_R, D = MK_SHAPE_GU_D; };      // GU: R/2 gate + R/2 up rows
template <> struct TaskShape<6> { static constexpr int R = MK_SHAPE_DOWN_R, D = MK_SHAPE_DOWN_D; };  // DOWN
template <> struct TaskShape<7> { static constexpr int R = MK_SHAPE_LM_R, D = MK_SHAPE_LM_D; };      // LM head
static_assert(TaskShape<1>::R >= 2 && TaskShape<5>::R % 2 == 0, "QKV needs a RoPE pair; GU pairs gate and up rows");
constexpr int kRowsQkv = TaskShape<1>::R, kRowsO = TaskShape<4>::R, kRowsGuPerMatrix = TaskShape<5>::R / 2,
              kRowsDown = TaskShape<6>::R, kRowsLm = TaskShape<7>::R;

// One task.  Interpretation of a0..a3 by type:
//   QKV   a0 = matrix (0 q, 1 k, 2 v), a1 = first row, a2 = rows, a3 = RoPE pair offset (0 = none)
//          rows are {a1 + i} for i < a2 when a3 == 0, else the pair {a1, a1 + a3} (a2 == 2)
//   ATTN  a0 = KV group, a1 = split index
//   MERGE a0 = KV group
//   O, DOWN, LM  a1 = first row, a2 = rows
//   GU    a1 = first row, a2 = rows per matrix
struct alignas(16) Task {
  uint8_t type;
  uint8_t page;          // LDS page of the staged input, kNone8 if none
  uint16_t layer;
  uint16_t in_event;     // event waited on, kNone16 if none
  uint16_t out_event;    // event signalled, kNone16 if none
  uint32_t in_count;     // signals on in_event per step (threshold = in_count * epoch)
  uint16_t stage;        // stage_key of the staged input, 0 if none
  uint16_t batch;        // batch row
  uint16_t local_slot;   // per-CU LDS counter used to aggregate out_event
  uint16_t local_count;  // tasks of this CU that signal out_event in one step
  uint32_t id;           // global task id (topological order)
  int32_t a0, a1, a2, a3;
};
static_assert(sizeof(Task) == 48, "Task layout");

// Launch arguments of a single-sequence GEMV operator kernel: the layer's
// weight matrices (QKV: q, k, v; GU: gate, up; O, DOWN, LM: w[0]) and the
// operator's task count.  The kernel derives task t from t itself
// (op_task_fields), so starting a weight stream takes no table lookups.
struct OpArgs {
  const uint16_t* w[3];
  const uint16_t* gain;  // RMSNorm gain of the staged input, null if it is not normalised
  int32_t layer;
  int32_t count;
  int32_t merge;         // O-projection: stage the input by merging the attention split records
};

#if defined(__HIPCC__)
#define MK_HD __host__ __device__
#else
#define MK_HD
#endif

// Task t of the single-sequence operator `type` (QKV, O, GU, DOWN, LM) of
// `layer`, in the order the graph builder emits them: QKV = the q RoPE pairs
// (head-major, pair i = rows i and i + hd/2), then the k pairs, then the v
// rows in runs of kRowsQkv; the others = runs of their row count.  Fields
// other than type, layer, stage, batch and a0..a3 are left zero.
MK_HD inline Task op_task_fields(int type, int layer, int t, int H, int nq, int nkv, int hd, int F, int V, int L) {
  Task d{};
  d.type = (uint8_t)type;
  d.page = kNone8;
  d.layer = (uint16_t)layer;
  d.in_event = kNone16;
  d.out_event = kNone16;
  d.batch = 0;
  auto rows = [](int t, int per, int n, Task& d) {
    d.a1 = t * per;
    d.a2 = n - d.a1 < per ? n - d.a1 : per;
  };
  switch (type) {
    case TT_QKV: {
      d.stage = stage_key(SK_ATTN_NORM, layer);
      const int half = hd / 2, pq = nq * half, pk = nkv * half;
      if (t < pq + pk) {
        const int u = t < pq ? t : t - pq;
        d.a0 = t < pq ? 0 : 1;
        d.a1 = (u / half) * hd + u % half;
        d.a2 = 2;
        d.a3 = half;
      } else {
        d.a0 = 2;
        rows(t - pq - pk, kRowsQkv, nkv * hd, d);
      }
      break;
    }
    case TT_O: d.stage = stage_key(SK_O_IN, layer); rows(t, kRowsO, H, d); break;
    case TT_GU: d.stage = stage_key(SK_FFN_NORM, layer); rows(t, kRowsGuPerMatrix, F, d); break;
    case TT_DOWN: d.stage = stage_key(SK_H, layer); rows(t, kRowsDown, H, d); break;
    case TT_LM: d.layer = (uint16_t)L; d.stage = stage_key(SK_FINAL_NORM, L); rows(t, kRowsLm, V, d); break;
    default: d.layer = (uint16_t)L; break;
  }
  return d;
}

// Device-visible description of a handle: shapes, weights, buffers, tables.
struct Params {
  // shape
  int32_t L, H, nq, nkv, hd, F, V, B, max_seq, split, nsplit, tied;
  int32_t kv_f32;       // KV cache element type: 0 bf16, 1 fp32
  float eps;
  int32_t ncu;          // persistent grid
  uint32_t timeout_ticks;   // wall-clock limit of any single wait
  uint32_t spin_limit;      // iteration limit of any single wait (backstop if the clock stalls)
  uint32_t shuffle_seed;    // nonzero: the megakernel rotates each operator's task dealing (MK_FLAG_SHUFFLE)
  uint32_t o_delay_ticks;   // megakernel: clock ticks the O projection's prefetch waits after the local QKV tasks
  // weights (bf16)
  const uint16_t* embed;
  const uint16_t* lm_head;
  const uint16_t* final_norm;
  const uint16_t* const* attn_norm;
  const uint16_t* const* wq;
  const uint16_t* const* wk;
  const uint16_t* const* wv;
  const uint16_t* const* wo;
  const uint16_t* const* ffn_norm;
  const uint16_t* const* w_gate;
  const uint16_t* const* w_up;
  const uint16_t* const* w_down;
  // KV cache [L][B][nkv][max_seq][hd], bf16 or fp32 (kv_f32)
  void* kcache;
  void* vcache;
  // fp32 activations (one buffer per layer, each written once per step)
  float* xs;         // [L+1][B][H]   x_{l+1} = output of layer l (x_0 unused: embedding row)
  float* xmid;       // [L][B][H]
  float* q;          // [L][B][nq*hd] (rotated)
  float* attn_part;  // [L][B][nkv][nsplit][G][hd + 2]  (o[hd], m, l)
  float* attn_out;   // [L][B][nq*hd]
  float* h;          // [L][B][F]
  // bf16 MFMA operands of the batched path, each value v as a pair of planes
  // hi = bf16(v), lo = bf16(v - hi) ([2][Bp][K]; rows B..Bp-1 stay zero); null when B == 1
  uint16_t* ax;      // K = H:      normalised input of QKV, gate/up and the LM head
  uint16_t* ao;      // K = nq*hd:  attention output
  uint16_t* ah;      // K = F:      SwiGLU output
  int32_t Bp;        // operand rows: B rounded up to 16, 32 or 64
  float* bpart;      // split-K partial sums of the batched projections
  unsigned long long* lm_part;  // [B] running argmax key (ordered value, ~index), cleared by the argmax task
  uint32_t* attn_count;         // [B][nkv] split workgroups finished this launch (fused merge), reset by the last
  const float* rope_cos;  // [max_seq][hd/2]
  const float* rope_sin;
  // task tables
  const Task* tasks;        // persistent: grouped by CU queue
  const int32_t* queue_off; // [ncu + 1]
  uint32_t* events;
  uint32_t* status;         // [16]: 0 abort flag, 1 error code, 2 cu, 3 task id, 4 event, 5 value, 6 need,
                            //       7 waiter (0 scheduler event, 1 scheduler page, 2 worker), 8 frontier, 9 ticket
  unsigned long long* trace;  // optional per-task timestamps
  int32_t trace_cap;
  int32_t trace_op;           // per-operator kernels: (type << 16) | layer whose waves log timestamps, -1 none
  // debug (mk_t_op_raw): when raw_out is set, a per-operator GEMV kernel
  // stages raw_in unnormalised and writes its raw dot products to raw_out
  // instead of running its epilogues
  const float* raw_in;
  float* raw_out;
};

// Per-launch arguments.
struct Step {
  uint32_t epoch;    // 1 for the first step after create/reset, +1 per launch
  int32_t pos;       // position written by this step (attention covers 0..pos)
  const int32_t* tokens;  // token of batch row b at tokens[b * tok_stride]
  int32_t tok_stride;
  int32_t* out;      // [B] greedy ids
  float* logits;     // [B][V] or null
  // megakernel only: steps run by this launch (epochs epoch + i, positions
  // pos + i); step i reads its token at tokens + i * tok_step, or, with
  // tok_step 0 and i > 0, takes the previous step's greedy id; it writes its
  // id to out + i * out_step; the logits are the last step's
  int32_t nsteps, tok_step, out_step;
};

// LDS header of the persistent and per-operator kernels (followed by the
// activation pages and the per-wave attention scratch).
struct Lds {
  uint32_t frontier, ticket, abort, pad0;
  uint32_t page_done[2];
  uint32_t pad1[2];
  uint32_t slot[kLocalSlots];
  unsigned long long lm_best[kMaxBatch];
};

// ---- persistent megakernel (one workgroup per CU, fixed wave roles) ----
constexpr int kMegaStagers = 4;   // waves that stage operator inputs and run attention, merges, argmax
constexpr int kMegaCompute = 4;   // waves that stream weights (the GEMV tasks), four tasks in flight each
constexpr int kMegaWaves = kMegaStagers + kMegaCompute;
constexpr int kMegaTraceSlots = kMegaCompute + 10;  // timestamps per (operator, workgroup) when tracing
// Microseconds the compute waves hold back the O projection's weight prefetch
// after their QKV tasks (8B shape, 256 steps: 0 us 3.154, 3 us 3.127, 6 us
// 3.133, 8 us 3.175 ms/token).
constexpr double kMegaOPrefetchDelayUs = 3.0;

// Buffers through which workgroups hand values to each other.  Each element
// is a 64-bit word: fp32 value bits in the low half, the epoch of the step
// that wrote it in the high half (the dependency signal).
struct MegaBufs {
  uint64_t* x;       // [L+1][H] residual stream after layer l-1 (row 0 unused: the embedding row)
  uint64_t* xmid;    // [L][H] residual after attention
  uint64_t* qkv;     // [L][(nq + 2 nkv) hd] rotated q, rotated k, v of the current position
  uint64_t* rec;     // [L][nkv][nsplit][G][hd + 2] attention split records (o[hd], m, l)
  uint64_t* attn;    // [L][nq hd] merged attention output
  uint64_t* h;       // [L][F] SwiGLU output
  uint64_t* key;     // [ncu] each workgroup's LM-head argmax key (epoch mod 2^15 in the low bits)
  uint64_t* tok;     // [1] the greedy id of the last step, tagged (epoch << 32 | id): the next step's input
  uint32_t* host_abort;          // host-mapped word: nonzero makes every wait give up
  unsigned long long* trace;     // optional [ops][ncu][kMegaTraceSlots] timestamps, null if off
};

// LDS header of the megakernel (followed by the two input pages, the
// residual copy, the RoPE angles, the compute waves' results and the stager
// waves' query buffers).
struct alignas(16) MegaLds {
  uint32_t ready[2];   // page p holds the input of operator ready[p] - 1
  uint32_t done[2];    // compute-wave completions of the operators on page p (cumulative)
  uint32_t pool[2];    // task pool counter of the operator on page p
  uint32_t ssync;      // stager rendezvous counter (cumulative)
  uint32_t abort;      // nonzero: every wave of the workgroup stops
  uint32_t lm_done;    // compute waves done with the LM head
  uint32_t pad[3];
  float red[kMegaStagers];     // stagers' partial sums of squares
  unsigned long long lm_best;  // best LM-head key of the workgroup
  unsigned long long pad2;
};

// Input pages of the megakernel: page 0 holds the hidden-size inputs (QKV,
// gate/up, LM head), page 1 the attention output and the SwiGLU output (O,
// down); floats each, rounded to 8.
MK_HD inline void mega_pages(int H, int qd, int F, int* pf0, int* pf1) {
  *pf0 = (H + 7) & ~7;
  *pf1 = ((qd > F ? qd : F) + 7) & ~7;
}

// Status codes latched by the kernel.
enum : uint32_t { ST_OK = 0, ST_TIMEOUT = 1, ST_NONFINITE = 2, ST_BADTOKEN = 3, ST_LDS = 4 };
constexpr int kStatusWords = 16;
constexpr uint32_t kLdsMagic = 0x4D4B4C44u;

}  // namespace mk
