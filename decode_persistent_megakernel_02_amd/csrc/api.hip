// Host implementation of the C ABI (include/mk.h, include/mk_debug.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <thread>
#include <cmath>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include <rocblas/rocblas.h>

#include "graph.h"
#include "kernels.h"
#include "mk.h"
#include "mk_debug.h"
#include "prefill.h"

using namespace mk;

namespace {

thread_local std::string g_err;

mk_status fail(mk_status s, const std::string& m) {
  g_err = m;
  return s;
}

#define HIP_TRY(x)                                                                              \
  do {                                                                                          \
    hipError_t e_ = (x);                                                                        \
    if (e_ != hipSuccess) return fail(MK_ERR_HIP, std::string(#x) + ": " + hipGetErrorString(e_)); \
  } while (0)

int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Positions per attention split when several sequences share a step: the
// (sequence, KV head) pairs already widen the grid.  Up to 1024 positions the
// whole context is one split (no merge launch; 70B shape, 64 sequences of
// 640: 58 against 69 + 8 us per layer).  Longer contexts use 512-position
// splits (8B shape, 8 sequences of 4K: 5.68 against 5.78 ms/step for 128),
// or the shortest multiple of 64 up to 1024 that keeps the workgroups within
// two per CU, one round of them: with 9 splits of 512 positions the last 64 of
// 576 workgroups ran in a second round (same workload: 31.3 + 6.0 us per
// layer, 8 splits of 576: 28.0 + 5.5).
int batched_split(int max_seq, int B, int nkv, int ncu) {
  if (max_seq <= 1024) return max_seq;
  for (int split = 512; split <= 1024; split += 64)
    if ((int64_t)B * nkv * ((max_seq + split - 1) / split) <= 2 * ncu) return split;
  return 512;
}


// Positions per attention split of the megakernel.  A (KV head, split) unit
// runs on the kMegaStagers stager waves of one workgroup, each taking whole
// position blocks of AttnGeom::NP positions; the split is the fewest such
// rounds of blocks that keep the units within one per workgroup.
int mega_block(int hd, bool f32) { return kWave / (hd / (f32 ? 16 : 32)); }
int mega_split(int max_seq, int nkv, int ncu, int hd, bool f32) {
  const int round = kMegaStagers * mega_block(hd, f32);
  for (int split = round;; split += round)
    if ((int64_t)nkv * ((max_seq + split - 1) / split) <= ncu || split >= kMaxSplit) return std::min(split, kMaxSplit);
}

// The megakernel instance for a shape: exact (no clamped loads) when every
// GEMV operator's K is a multiple of 2048 and the task order is not shuffled
// (only the generic instances rotate it); by head_dim, cache type and query
// heads per KV head (1, 2, 4, 8).
const void* mega_kernel(int H, int qd, int F, int hd, bool f32, int G, bool shuffle) {
  const bool exact = H % 2048 == 0 && qd % 2048 == 0 && F % 2048 == 0 && G == 4 && !shuffle;
#define MK_K(X, HD, KN, G) reinterpret_cast<const void*>(&mk_mega_##X##_##HD##_##KN##_g##G)
  if (exact) {
    if (hd == 64) return f32 ? MK_K(x, 64, f32, 4) : MK_K(x, 64, bf16, 4);
    return f32 ? MK_K(x, 128, f32, 4) : MK_K(x, 128, bf16, 4);
  }
  static const void* const k[2][2][4] = {
      {{MK_K(n, 64, bf16, 1), MK_K(n, 64, bf16, 2), MK_K(n, 64, bf16, 4), MK_K(n, 64, bf16, 8)},
       {MK_K(n, 64, f32, 1), MK_K(n, 64, f32, 2), MK_K(n, 64, f32, 4), MK_K(n, 64, f32, 8)}},
      {{MK_K(n, 128, bf16, 1), MK_K(n, 128, bf16, 2), MK_K(n, 128, bf16, 4), MK_K(n, 128, bf16, 8)},
       {MK_K(n, 128, f32, 1), MK_K(n, 128, f32, 2), MK_K(n, 128, f32, 4), MK_K(n, 128, f32, 8)}}};
#undef MK_K
  const int gi = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : G == 8 ? 3 : -1;
  return gi < 0 ? nullptr : k[hd == 128 ? 1 : 0][f32 ? 1 : 0][gi];
}

// Batch tiles (16 rows each) of the batched projections: 1, 2 or 4.
int batch_tiles(int B) { return B <= 16 ? 1 : B <= 32 ? 2 : 4; }

std::string check_config(const mk_config* c) {
  if (!c) return "config is NULL";
  if (c->abi_version != MK_ABI_VERSION) return "abi_version mismatch";
  if (c->n_layers < 1 || c->hidden < 8 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->ffn < 8 || c->vocab < 1)
    return "non-positive model dimension";
  if (c->head_dim != 64 && c->head_dim != 128) return "head_dim must be 64 or 128";
  if (c->n_q_heads % c->n_kv_heads) return "n_q_heads must be a multiple of n_kv_heads";
  if (c->n_q_heads / c->n_kv_heads > kMaxGqa) return "at most 8 query heads per KV head";
  if (c->hidden % 8 || c->ffn % 8 || (c->n_q_heads * c->head_dim) % 8)
    return "hidden, ffn and n_q_heads*head_dim must be multiples of 8";
  if (c->max_batch < 1 || c->max_batch > kMaxBatch) return "max_batch must be in [1, 64]";
  if (c->max_seq < 1) return "max_seq must be >= 1";
  if (c->mode != MK_MODE_MEGAKERNEL && c->mode != MK_MODE_PER_OP) return "unknown mode";
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) return "rms_eps must be >= 0 and rope_theta > 0";
  if (c->attn_split < 0 || c->attn_split > kMaxSplit) return "attn_split must be in [0, 4096]";
  if (c->num_cus < 0) return "num_cus must be >= 0";
  if ((int64_t)c->vocab * c->hidden >= (1ll << 40)) return "vocab * hidden too large";
  if ((c->flags & MK_FLAG_SHUFFLE) && (c->mode != MK_MODE_MEGAKERNEL || c->max_batch != 1))
    return "MK_FLAG_SHUFFLE reorders the megakernel's task dealing (megakernel mode, max_batch 1)";
  if (c->flags & MK_FLAG_TILED_WEIGHTS) {
    if (c->max_batch < 2) return "tiled weights are read by the batched path only (max_batch >= 2)";
    const int qd = c->n_q_heads * c->head_dim, kd = c->n_kv_heads * c->head_dim;
    if (c->hidden % 32 || c->ffn % 32 || qd % 32 || kd % 16 || (!c->tie_embeddings && c->vocab % 16))
      return "tiled weights need row counts that are multiples of 16 and column counts that are multiples of 32";
  }
  return "";
}

GraphConfig graph_config(const mk_config* c, int ncu) {
  GraphConfig g;
  g.L = c->n_layers; g.H = c->hidden; g.nq = c->n_q_heads; g.nkv = c->n_kv_heads; g.hd = c->head_dim;
  g.F = c->ffn; g.V = c->vocab; g.B = c->max_batch; g.max_seq = c->max_seq;
  g.split = c->attn_split ? c->attn_split
            : c->max_batch > 1 ? batched_split(c->max_seq, c->max_batch, c->n_kv_heads, ncu)
            : c->mode == MK_MODE_MEGAKERNEL ? mega_split(c->max_seq, c->n_kv_heads, ncu, c->head_dim, c->kv_fp32 != 0)
                                            : auto_split(c->max_seq);
  g.ncu = ncu;
  return g;
}

int64_t task_weight_bytes(const GraphConfig& c, const Task& t) {
  switch (t.type) {
    case TT_QKV: return (int64_t)t.a2 * c.H * 2;
    case TT_O: return (int64_t)t.a2 * c.nq * c.hd * 2;
    case TT_GU: return (int64_t)2 * t.a2 * c.H * 2;
    case TT_DOWN: return (int64_t)t.a2 * c.F * 2;
    case TT_LM: return (int64_t)t.a2 * c.H * 2;
    default: return 0;
  }
}

// The per-operator kernels derive their tasks arithmetically
// (op_task_fields); they must be the tasks the graph builder emitted.
std::string check_op_tasks(const Graph& g) {
  const GraphConfig& c = g.cfg;
  for (size_t s = 0; s + 1 < g.stage_begin.size(); ++s) {
    const int type = g.stage_type[s], b0 = g.stage_begin[s], n = g.stage_begin[s + 1] - b0;
    if (type != TT_QKV && type != TT_O && type != TT_GU && type != TT_DOWN && type != TT_LM) continue;
    for (int i = 0; i < n; ++i) {
      const Task& t = g.tasks[b0 + i];
      const Task d = op_task_fields(type, t.layer, i, c.H, c.nq, c.nkv, c.hd, c.F, c.V, c.L);
      if (d.type != t.type || d.layer != t.layer || d.stage != t.stage || d.batch != t.batch || d.a0 != t.a0 ||
          d.a1 != t.a1 || d.a2 != t.a2 || d.a3 != t.a3)
        return "operator task formula differs from the graph at stage " + std::to_string(s) + ", task " +
               std::to_string(i);
    }
  }
  return "";
}

}  // namespace

struct mk_handle {
  mk_config cfg{};
  hipStream_t stream = nullptr;
  int device = 0;
  Graph graph;         // single sequence: the task graph (per-CU queues, events)
  BatchedGraph bgraph; // B >= 2: the stages of the matrix-core launch plan
  Params P{};
  std::vector<void*> allocs;
  int page_floats = 0, lds_mega = 0;  // megakernel: input page floats, LDS bytes
  MegaBufs mega{};                    // megakernel: tagged hand-over buffers
  const void* mega_fn = nullptr;      // megakernel: the instance for this shape
  uint32_t* host_abort = nullptr;     // megakernel: host-mapped abort word (hipHostMalloc)
  int64_t mega_trace_words = 0;       // megakernel: words of the timestamp buffer (0: off)
  int pending = 0;                    // launches since the last synchronize (host watchdog)
  int op_page[9] = {0}, op_lds[9] = {0}, op_grid_cap[9] = {0}, op_sf[9] = {0};  // per task type
  int op_grid[9] = {0};  // grid of the last launch of each GEMV operator
  bool op_exact[9] = {false};
  bool batched = false;                 // B > 1: matrix-core projections (batched.hip)
  int length = 0, batch = 0;
  uint32_t epoch = 0;
  bool poisoned = false;
  int32_t* d_tok_scratch = nullptr;
  Step* d_step = nullptr;               // per-step arguments, written by mk_set_step
  int attn_lds = 0;                     // per-op split attention kernel
  int attn_full_lds = 0;                // whole-context attention kernel
  hipStream_t cap_stream = nullptr;     // private stream used to capture the step graph
  hipGraph_t step_graph = nullptr;
  hipGraphExec_t graph_exec = nullptr;
  float* act = nullptr;
  int64_t act_floats = 0;
  double ticks_per_us = 100.0;
  // optional HIP-event timing of selected operators (per-op mode)
  uint32_t timed_mask = 0;
  std::vector<hipEvent_t> ev_pool;  // pairs: [2i] start, [2i+1] end
  std::vector<int> ev_type;
  int ev_used = 0;
  std::vector<const void*> host_w;      // [9][L] layer pointer tables (as in P), host copy
  // back-to-back replay of one operator's launches (mk_time_op_replay)
  int only_type = -1, replayed = 0;
  hipEvent_t rep_ev[2] = {nullptr, nullptr};
  // batched prefill (MK_FLAG_BATCHED_PREFILL): matrix-core projections through rocBLAS
  rocblas_handle blas = nullptr;
  int pf_rows = 0, pf_cap = 0;          // rows (sequence x position) per chunk; its allocated maximum
  float* pf_x = nullptr;                // [rows][H] residual stream of the chunk
  float* pf_y = nullptr;                // [rows][max(qd + 2 kd, 2F, H)] projection outputs
  uint16_t* pf_ops = nullptr;           // [2][rows][K] bf16 operand of one projection: high parts, then low
  float* pf_logits = nullptr;           // [2][max_batch][V] LM-head outputs of the two operand parts

  template <class T>
  mk_status alloc(T** p, int64_t count) {
    void* q = nullptr;
    const size_t bytes = std::max<int64_t>(count, 1) * sizeof(T);
    if (hipMalloc(&q, bytes) != hipSuccess) {
      (void)hipGetLastError();
      return fail(MK_ERR_OUT_OF_MEMORY, "hipMalloc of " + std::to_string(bytes) + " bytes failed");
    }
    allocs.push_back(q);
    *p = static_cast<T*>(q);
    return MK_OK;
  }
  ~mk_handle() {
    if (blas) (void)rocblas_destroy_handle(blas);
    if (host_abort) (void)hipHostFree(host_abort);
    if (graph_exec) (void)hipGraphExecDestroy(graph_exec);
    if (step_graph) (void)hipGraphDestroy(step_graph);
    if (cap_stream) (void)hipStreamDestroy(cap_stream);
    for (hipEvent_t e : ev_pool) (void)hipEventDestroy(e);
    for (hipEvent_t e : rep_ev)
      if (e) (void)hipEventDestroy(e);
    for (void* p : allocs) (void)hipFree(p);
  }
};

#define MK_TRY(x)                     \
  do {                                \
    mk_status s_ = (x);               \
    if (s_ != MK_OK) return s_;       \
  } while (0)

namespace {

// The per-operator kernel of a task type; `exact` selects the variant for K a
// multiple of 512 whose 512-column chunk count is a multiple of D.
const void* op_kernel(int type, bool exact = false) {
  if (exact) {
    switch (type) {
      case TT_QKV: return reinterpret_cast<const void*>(&mk_op_qkv_x);
      case TT_O: return reinterpret_cast<const void*>(&mk_op_o_x);
      case TT_GU: return reinterpret_cast<const void*>(&mk_op_gu_x);
      case TT_DOWN: return reinterpret_cast<const void*>(&mk_op_down_x);
      case TT_LM: return reinterpret_cast<const void*>(&mk_op_lm_x);
      default: break;
    }
  }
  switch (type) {
    case TT_QKV: return reinterpret_cast<const void*>(&mk_op_qkv);
    case TT_O: return reinterpret_cast<const void*>(&mk_op_o);
    case TT_GU: return reinterpret_cast<const void*>(&mk_op_gu);
    case TT_DOWN: return reinterpret_cast<const void*>(&mk_op_down);
    case TT_LM: return reinterpret_cast<const void*>(&mk_op_lm);
    default: return reinterpret_cast<const void*>(&mk_op_argmax);
  }
}

mk_status device_facts(int* ncu, double* ticks_per_us, int* max_lds) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  int n = 0, khz = 0, lds = 0;
  HIP_TRY(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev));
  HIP_TRY(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev));
  HIP_TRY(hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
  int optin = 0;
  if (hipDeviceGetAttribute(&optin, hipDeviceAttributeSharedMemPerBlockOptin, dev) == hipSuccess && optin > lds)
    lds = optin;
  (void)hipGetLastError();
  if (ncu) *ncu = n;
  if (ticks_per_us) *ticks_per_us = khz > 0 ? khz / 1000.0 : 100.0;
  if (max_lds) *max_lds = lds;
  return MK_OK;
}

bool fused_merge(const mk_handle* h) { return (h->cfg.flags & MK_FLAG_FUSED_MERGE) != 0; }
// A context that fits one split runs as one workgroup per (sequence, KV head)
// that writes the final output (no merge launch).  Forcing that shape on
// longer contexts measured slower: at the 8B shape, batch 1, 37 against 21 us
// per layer (8 CUs busy), and at the 70B shape, 64 sequences, 100 against 73.
bool single_split(const mk_handle* h) { return h->P.nsplit == 1; }
// Single sequence, split attention, no fused merge: the O-projection merges
// the split records while it stages its input (one launch fewer per layer).
bool merge_in_o(const mk_handle* h) { return !h->batched && !fused_merge(h) && !single_split(h); }

// Attention kernels by cache element type and query heads per KV group
// (compile-time group sizes 1, 2, 4, 8; other sizes use the run-time variant).
const void* attn_split_kernel(bool f32, int G) {
#define MK_PICK(KN)                                                                    \
  switch (G) {                                                                         \
    case 1: return reinterpret_cast<const void*>(&mk_op_attn_split_##KN##_g1);        \
    case 2: return reinterpret_cast<const void*>(&mk_op_attn_split_##KN##_g2);        \
    case 4: return reinterpret_cast<const void*>(&mk_op_attn_split_##KN##_g4);        \
    case 8: return reinterpret_cast<const void*>(&mk_op_attn_split_##KN##_g8);        \
    default: return reinterpret_cast<const void*>(&mk_op_attn_split_##KN##_g0);       \
  }
  if (f32) MK_PICK(f32) else MK_PICK(bf16)
#undef MK_PICK
}
const void* attn_full_kernel(bool f32, int G) {
#define MK_PICK(KN)                                                                    \
  switch (G) {                                                                         \
    case 1: return reinterpret_cast<const void*>(&mk_op_attn_full_##KN##_g1);         \
    case 2: return reinterpret_cast<const void*>(&mk_op_attn_full_##KN##_g2);         \
    case 4: return reinterpret_cast<const void*>(&mk_op_attn_full_##KN##_g4);         \
    case 8: return reinterpret_cast<const void*>(&mk_op_attn_full_##KN##_g8);         \
    default: return reinterpret_cast<const void*>(&mk_op_attn_full_##KN##_g0);        \
  }
  if (f32) MK_PICK(f32) else MK_PICK(bf16)
#undef MK_PICK
}

// Batched projection kernels by operator (QKV, O, GU, DOWN, LM), batch tiles
// (1, 2, 4), weight layout (row-major, tiled) and row groups per wave (1; 2
// for 4 batch tiles).
const void* bgemm_kernel(int type, int bt, bool tiled, int gpw) {
  const int i = gpw == 2 ? 3 : bt == 1 ? 0 : bt == 2 ? 1 : 2;
#define MK_K(op) {reinterpret_cast<const void*>(&mk_b_##op##_b1), reinterpret_cast<const void*>(&mk_b_##op##_b2), \
                   reinterpret_cast<const void*>(&mk_b_##op##_b4), reinterpret_cast<const void*>(&mk_b_##op##_b4_g2)}, \
                  {reinterpret_cast<const void*>(&mk_b_##op##_b1_t), reinterpret_cast<const void*>(&mk_b_##op##_b2_t), \
                   reinterpret_cast<const void*>(&mk_b_##op##_b4_t), reinterpret_cast<const void*>(&mk_b_##op##_b4_t_g2)}
  static const void* const k[5][2][4] = {{MK_K(qkv)}, {MK_K(o)}, {MK_K(gu)}, {MK_K(down)}, {MK_K(lm)}};
#undef MK_K
  const int row = type == TT_QKV ? 0 : type == TT_O ? 1 : type == TT_GU ? 2 : type == TT_DOWN ? 3 : 4;
  return k[row][tiled ? 1 : 0][i];
}
int bgemm_lds(int bt) { return b_lds_bytes(bt) + kMaxBatch * 8; }

// Row groups of a batched projection (one per wave: two 16-row tiles), and K.
int bgemm_groups(const Params& P, int type) {
  switch (type) {
    case TT_QKV: return (P.nq + 2 * P.nkv) * P.hd / 32;
    case TT_O: case TT_DOWN: return (P.H + 31) / 32;
    case TT_GU: return (P.F + 15) / 16;
    default: return (P.V + 31) / 32;
  }
}
// Row groups per wave of a batched projection: two with 4 batch tiles when
// that still leaves at least half a workgroup per CU without splitting K
// (measured at the 70B shape, 64 sequences: gate/up 233 -> 211 us, but the
// O-projection and down, with 8x fewer groups, got slower).
int bgemm_gpw(const Params& P, int type) {
  return batch_tiles(P.B) == 4 && bgemm_groups(P, type) / (2 * kBgemmWaves) >= P.ncu / 2 ? 2 : 1;
}
// Workgroups along the rows of a batched projection.
int bgemm_blocks(const Params& P, int type) {
  const int per = kBgemmWaves * bgemm_gpw(P, type);
  return (bgemm_groups(P, type) + per - 1) / per;
}
int bgemm_k(const Params& P, int type) { return type == TT_O ? P.nq * P.hd : type == TT_DOWN ? P.F : P.H; }

// Splits of K for a batched projection: enough workgroups for the target
// below, whole activation chunks per split, none empty; the LM head is not
// split (its argmax runs in the epilogue).
int bgemm_splits(const Params& P, int type, int ncu) {
  if (type == TT_LM) return 1;
  const int bt = batch_tiles(P.B), kc = kBChunkCols[bt];
  const int ngx = bgemm_blocks(P, type);
  const int nch = (bgemm_k(P, type) + kc - 1) / kc;
  // Workgroups to aim for: two per CU where each weight byte carries the most
  // matrix-core and LDS work (64 sequences, one row group per wave), one
  // elsewhere, which halves the partial sums the finishing launch adds.
  // Measured per operator at the 8B shape with 8 sequences and the 70B shape
  // with 64; three per CU was slower everywhere.
  // Two per CU is also as many of those workgroups as the CUs hold at once
  // (LDS), so there the count rounds down: a few more would run in a second
  // round (70B shape, 64 sequences: QKV in 7 splits was 560 workgroups).
  // With one batch tile (up to 16 sequences) it rounds down too: at the 8B
  // shape with 8 sequences gate/up then runs unsplit (224 workgroups, no
  // finishing launch) and QKV in 5 splits instead of 6 (240 workgroups, not
  // 288): 4.710 -> 4.581 ms/step.  Rounding down at four batch tiles with two
  // row groups per wave (the 70B shape's gate/up, 64 sequences: one split
  // instead of two) was slower: 33.07 -> 33.85 ms/step.
  const bool two = bt == 4 && bgemm_gpw(P, type) == 1;
  const int target = (two ? 2 : 1) * ncu;
  const bool round_down = two || bt == 1;
  int ks = std::max(1, std::min(nch, round_down ? target / ngx : (target + ngx - 1) / ngx));
  const int per = (nch + ks - 1) / ks;
  return (nch + per - 1) / per;
}

// The tiling of every batched projection, from the helpers above (the same
// values the launches use), for the batched task graph.
BatchedConfig batched_config(const mk_config* c, int ncu, int nsplit) {
  Params P{};
  P.L = c->n_layers; P.H = c->hidden; P.nq = c->n_q_heads; P.nkv = c->n_kv_heads; P.hd = c->head_dim;
  P.F = c->ffn; P.V = c->vocab; P.B = c->max_batch; P.ncu = ncu; P.nsplit = nsplit;
  BatchedConfig bc{};
  bc.L = P.L; bc.H = P.H; bc.nq = P.nq; bc.nkv = P.nkv; bc.hd = P.hd; bc.F = P.F; bc.V = P.V; bc.B = P.B;
  bc.nsplit = nsplit;
  bc.fused_merge = (c->flags & MK_FLAG_FUSED_MERGE) != 0;
  for (int t : {TT_QKV, TT_O, TT_GU, TT_DOWN, TT_LM}) {
    BGemm& m = bc.gemm[t];
    m.groups = bgemm_groups(P, t);
    m.per_block = kBgemmWaves * bgemm_gpw(P, t);
    m.blocks = bgemm_blocks(P, t);
    m.splits = bgemm_splits(P, t, ncu);
    m.chunk_cols = kBChunkCols[batch_tiles(P.B)];
    m.K = bgemm_k(P, t);
    m.N = t == TT_QKV ? (P.nq + 2 * P.nkv) * P.hd : t == TT_GU ? P.F : t == TT_LM ? P.V : P.H;
  }
  return bc;
}

const void* bfin_kernel(int type) {
  switch (type) {
    case TT_QKV: return reinterpret_cast<const void*>(&mk_b_fin_qkv);
    case TT_O: return reinterpret_cast<const void*>(&mk_b_fin_o);
    case TT_GU: return reinterpret_cast<const void*>(&mk_b_fin_gu);
    default: return reinterpret_cast<const void*>(&mk_b_fin_down);
  }
}

// Whether the batched projection `type` reads tiled weights (the LM head of a
// tied model reads the row-major embedding table).
bool tiled_ops(const mk_handle* h, int type) {
  return (h->cfg.flags & MK_FLAG_TILED_WEIGHTS) && !(type == TT_LM && h->P.tied);
}

// One step of the batched path: per layer norm, QKV, attention, merge, O,
// norm, gate/up, down; then the final norm, the LM head and the argmax.
// Timed launches are bracketed by events (type 0 = the norms).
mk_status enqueue_batched(mk_handle* h, hipStream_t st, bool timed_ok) {
  Params Pc = h->P;
  const Step* sp = h->d_step;
  const int bt = batch_tiles(Pc.B);
  auto launch = [&](int type, const void* fn, dim3 grid, dim3 block, void** args, size_t lds) -> mk_status {
    if (h->only_type >= 0) {
      if (type != h->only_type) return MK_OK;
      ++h->replayed;
    }
    const bool timed = timed_ok && ((h->timed_mask >> type) & 1) && 2 * (h->ev_used + 1) <= (int)h->ev_pool.size();
    if (timed) HIP_TRY(hipEventRecord(h->ev_pool[2 * h->ev_used], st));
    HIP_TRY(hipLaunchKernel(fn, grid, block, args, lds, st));
    if (timed) {
      HIP_TRY(hipEventRecord(h->ev_pool[2 * h->ev_used + 1], st));
      h->ev_type[h->ev_used++] = type;
    }
    return MK_OK;
  };
  // One launch per stage of the batched task graph, its grid the stage's task
  // grid (validated at create against the buffers every stage reads and writes).
  const BatchedGraph& g = h->bgraph;
  for (const BStage& s : g.stages) {
    int layer = s.layer;
    switch (s.kind) {
      case BK_NORM: {
        int kind = s.sub;
        void* args[] = {&Pc, &sp, &layer, &kind};
        MK_TRY(launch(0, reinterpret_cast<const void*>(&mk_b_norm), dim3(s.gx), dim3(kNormThreads), args, 0));
        break;
      }
      case BK_GEMM: {
        void* args[] = {&Pc, &sp, &layer};
        const void* fn = bgemm_kernel(s.type, bt, tiled_ops(h, s.type), bgemm_gpw(Pc, s.type));
        MK_TRY(launch(s.type, fn, dim3(s.gx, s.gy), dim3(kBgemmWaves * kWave), args, (size_t)bgemm_lds(bt)));
        break;
      }
      case BK_FIN: {
        int k = g.cfg.gemm[s.type].splits;
        void* args[] = {&Pc, &sp, &layer, &k};
        MK_TRY(launch(s.type, bfin_kernel(s.type), dim3(s.gx), dim3(16 * Pc.Bp), args, 0));  // 16 * Bp <= 1024
        break;
      }
      case BK_ATTN_FULL: {
        void* args[] = {&Pc, &sp, &layer};
        MK_TRY(launch(TT_ATTN, attn_full_kernel(Pc.kv_f32, Pc.nq / Pc.nkv), dim3(s.gx),
                      dim3(kAttnFullWaves * kWave), args, (size_t)h->attn_full_lds));
        break;
      }
      case BK_ATTN: {
        int fuse = g.cfg.fused_merge ? 1 : 0;
        void* args[] = {&Pc, &sp, &layer, &fuse};
        MK_TRY(launch(TT_ATTN, attn_split_kernel(Pc.kv_f32, Pc.nq / Pc.nkv), dim3(s.gx), dim3(kAttnWaves * kWave),
                      args, (size_t)h->attn_lds));
        break;
      }
      case BK_MERGE: {
        if (s.gx == 0) break;  // merged by the attention launch's last workgroups
        int fuse = 0;
        void* args[] = {&Pc, &sp, &layer, &fuse};
        MK_TRY(launch(TT_MERGE, reinterpret_cast<const void*>(&mk_op_attn_merge), dim3(s.gx),
                      dim3((Pc.nq / Pc.nkv) * kWave), args, 0));
        break;
      }
      default: {
        void* args[] = {&Pc, &sp};
        MK_TRY(launch(TT_ARGMAX, reinterpret_cast<const void*>(&mk_b_argmax), dim3(1), dim3(kMaxBatch), args, 0));
        break;
      }
    }
  }
  return MK_OK;
}

// Launch arguments of the single-sequence operator `type` of `layer`.
OpArgs op_args(const mk_handle* h, int type, int layer, int count) {
  const int L = h->P.L;
  auto w = [&](int table) { return static_cast<const uint16_t*>(h->host_w[(size_t)table * L + layer]); };
  OpArgs A{};
  A.layer = layer;
  A.count = count;
  switch (type) {  // tables: attn_norm, wq, wk, wv, wo, ffn_norm, w_gate, w_up, w_down
    case TT_QKV: A.w[0] = w(1); A.w[1] = w(2); A.w[2] = w(3); A.gain = w(0); break;
    case TT_O: A.w[0] = w(4); break;
    case TT_GU: A.w[0] = w(6); A.w[1] = w(7); A.gain = w(5); break;
    case TT_DOWN: A.w[0] = w(8); break;
    case TT_LM: A.w[0] = h->P.tied ? h->P.embed : h->P.lm_head; A.gain = h->P.final_norm; break;
    default: break;
  }
  return A;
}

// Enqueue the operator launches of one step (kernel-per-operator mode) on `st`.
mk_status enqueue_ops(mk_handle* h, hipStream_t st, bool timed_ok) {
  if (h->batched) return enqueue_batched(h, st, timed_ok);
  const auto& g = h->graph;
  Params Pc = h->P;
  const Step* sp = h->d_step;
  for (size_t s = 0; s + 1 < g.stage_begin.size(); ++s) {
    const int b0 = g.stage_begin[s], count = g.stage_begin[s + 1] - b0;
    if (count <= 0) continue;
    const int type = g.stage_type[s];
    if (type == TT_MERGE && (fused_merge(h) || single_split(h) || merge_in_o(h))) continue;  // done elsewhere
    if (h->only_type >= 0) {
      if (type != h->only_type) continue;
      ++h->replayed;
    }
    const bool timed = timed_ok && ((h->timed_mask >> type) & 1) && 2 * (h->ev_used + 1) <= (int)h->ev_pool.size();
    if (timed) HIP_TRY(hipEventRecord(h->ev_pool[2 * h->ev_used], st));
    if (type == TT_ATTN || type == TT_MERGE) {
      int layer = g.tasks[b0].layer, fuse = fused_merge(h) ? 1 : 0;
      void* args[] = {&Pc, &sp, &layer, &fuse};
      if (type == TT_ATTN && single_split(h))
        HIP_TRY(hipLaunchKernel(attn_full_kernel(h->P.kv_f32, h->P.nq / h->P.nkv), dim3(h->P.B * h->P.nkv),
                                dim3(kAttnFullWaves * kWave), args, (size_t)h->attn_full_lds, st));
      else if (type == TT_ATTN)
        HIP_TRY(hipLaunchKernel(attn_split_kernel(h->P.kv_f32, h->P.nq / h->P.nkv),
                                dim3(h->P.B * h->P.nkv * h->P.nsplit), dim3(kAttnWaves * kWave), args,
                                (size_t)h->attn_lds, st));
      else
        HIP_TRY(hipLaunchKernel(reinterpret_cast<const void*>(&mk_op_attn_merge), dim3(h->P.B * h->P.nkv),
                                dim3((h->P.nq / h->P.nkv) * kWave), args, 0, st));
    } else {
      // a GEMV wave holds at most kMaxTasksPerWave results: keep the average at half of that
      const int min_grid = (count + kWaves * kMaxTasksPerWave / 2 - 1) / (kWaves * kMaxTasksPerWave / 2);
      const int grid = std::max(min_grid, std::min((count + kWaves - 1) / kWaves, h->op_grid_cap[type]));
      h->op_grid[type] = grid;
      OpArgs A = op_args(h, type, g.tasks[b0].layer, count);
      A.merge = type == TT_O && merge_in_o(h) ? 1 : 0;
      int opf = h->op_page[type];
      int osf = h->op_sf[type];
      void* args[] = {&Pc, &sp, &A, &opf, &osf};
      HIP_TRY(hipLaunchKernel(op_kernel(type, h->op_exact[type]), dim3(grid), dim3(kWaves * kWave), args,
                              (size_t)h->op_lds[type], st));
    }
    if (timed) {
      HIP_TRY(hipEventRecord(h->ev_pool[2 * h->ev_used + 1], st));
      h->ev_type[h->ev_used++] = type;
    }
  }
  return MK_OK;
}

// One single-sequence GEMV operator launch of `layer`, the shipped kernel and
// launch configuration, with the given Params (enqueue_ops' GEMV branch).
mk_status launch_op(mk_handle* h, const Params& Pin, int type, int layer, hipStream_t st) {
  const auto& g = h->graph;
  for (size_t s = 0; s + 1 < g.stage_begin.size(); ++s) {
    const int b0 = g.stage_begin[s], count = g.stage_begin[s + 1] - b0;
    if (count <= 0 || g.stage_type[s] != type || g.tasks[b0].layer != layer) continue;
    Params Pc = Pin;
    const Step* sp = h->d_step;
    const int min_grid = (count + kWaves * kMaxTasksPerWave / 2 - 1) / (kWaves * kMaxTasksPerWave / 2);
    const int grid = std::max(min_grid, std::min((count + kWaves - 1) / kWaves, h->op_grid_cap[type]));
    OpArgs A = op_args(h, type, layer, count);
    A.merge = 0;
    int opf = h->op_page[type];
    int osf = h->op_sf[type];
    void* args[] = {&Pc, &sp, &A, &opf, &osf};
    HIP_TRY(hipLaunchKernel(op_kernel(type, h->op_exact[type]), dim3(grid), dim3(kWaves * kWave), args,
                            (size_t)h->op_lds[type], st));
    return MK_OK;
  }
  return fail(MK_ERR_INVALID_ARG, "no such operator in the task graph");
}

// Capture one step's operator launches into a graph (once per handle).
mk_status build_step_graph(mk_handle* h) {
  if (h->graph_exec) return MK_OK;
  if (!h->cap_stream) HIP_TRY(hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking));
  HIP_TRY(hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal));
  mk_status st = enqueue_ops(h, h->cap_stream, false);
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamEndCapture(h->cap_stream, &graph);
  if (st != MK_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return st;
  }
  if (e != hipSuccess) return fail(MK_ERR_HIP, std::string("graph capture: ") + hipGetErrorString(e));
  h->step_graph = graph;
  HIP_TRY(hipGraphInstantiate(&h->graph_exec, h->step_graph, nullptr, nullptr, 0));
  return MK_OK;
}

mk_status launch_step(mk_handle* h, const Step& S) {
  const Params& P = h->P;
  if (h->cfg.flags & MK_FLAG_POISON) {
    hipLaunchKernelGGL(mk_fill_u32, dim3(1024), dim3(256), 0, h->stream, reinterpret_cast<uint32_t*>(h->act),
                       h->act_floats, 0xFFFFFFFFu);
    HIP_TRY(hipGetLastError());
  }
  if (h->cfg.mode == MK_MODE_MEGAKERNEL) {
    // One ordinary launch of one workgroup per CU (the LDS request keeps a
    // second one off each CU).  The kernel uses no grid-wide barrier, so it
    // needs no cooperative launch; every in-kernel wait is bounded, so a
    // workgroup that were not resident would end the step with
    // MK_ERR_TIMEOUT rather than hang it.
    Params Pc = P;
    MegaBufs Mc = h->mega;
    Step Sc = S;
    int pf = h->page_floats;
    void* args[] = {&Pc, &Mc, &Sc, &pf};
    HIP_TRY(hipLaunchKernel(h->mega_fn, dim3(P.ncu), dim3(kMegaWaves * kWave), args, (size_t)h->lds_mega, h->stream));
    h->pending += S.nsteps > 0 ? S.nsteps : 1;
    return MK_OK;
  }
  hipLaunchKernelGGL(mk_set_step, dim3(1), dim3(64), 0, h->stream, h->d_step, S);
  HIP_TRY(hipGetLastError());
  const bool eager = (h->cfg.flags & MK_FLAG_NO_GRAPH) || h->timed_mask != 0;
  if (eager) return enqueue_ops(h, h->stream, true);
  MK_TRY(build_step_graph(h));
  HIP_TRY(hipGraphLaunch(h->graph_exec, h->stream));
  return MK_OK;
}

}  // namespace

extern "C" {

const char* mk_last_error(void) { return g_err.c_str(); }

mk_status mk_device_info(int32_t* ncu, double* ticks_per_us, int32_t* max_lds) {
  int n = 0, l = 0;
  double t = 0;
  MK_TRY(device_facts(&n, &t, &l));
  if (ncu) *ncu = n;
  if (ticks_per_us) *ticks_per_us = t;
  if (max_lds) *max_lds = l;
  return MK_OK;
}

mk_status mk_create(const mk_config* cfg, const mk_weights* w, void* hip_stream, mk_handle** out) {
  g_err.clear();
  if (!out) return fail(MK_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  const std::string cerr = check_config(cfg);
  if (!cerr.empty()) return fail(MK_ERR_INVALID_ARG, cerr);
  if (!w || !w->embed || !w->final_norm || !w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo || !w->ffn_norm ||
      !w->w_gate || !w->w_up || !w->w_down)
    return fail(MK_ERR_INVALID_ARG, "weights: NULL pointer");
  if ((w->lm_head == nullptr) != (cfg->tie_embeddings != 0))
    return fail(MK_ERR_INVALID_ARG, "weights: lm_head must be NULL exactly when tie_embeddings is set");
  for (int l = 0; l < cfg->n_layers; ++l)
    if (!w->attn_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->ffn_norm[l] || !w->w_gate[l] ||
        !w->w_up[l] || !w->w_down[l])
      return fail(MK_ERR_INVALID_ARG, "weights: NULL pointer in layer " + std::to_string(l));
  if (cfg->mode == MK_MODE_MEGAKERNEL) {
    if (cfg->max_batch != 1)
      return fail(MK_ERR_UNSUPPORTED, "MK_MODE_MEGAKERNEL runs one sequence (max_batch 1); batched decode runs per operator");
    const int G = cfg->n_q_heads / cfg->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
      return fail(MK_ERR_UNSUPPORTED, "MK_MODE_MEGAKERNEL supports 1, 2, 4 or 8 query heads per KV head");
    if (cfg->vocab > (1 << 17)) return fail(MK_ERR_UNSUPPORTED, "MK_MODE_MEGAKERNEL supports vocab <= 131072");
    if (cfg->n_q_heads > 256) return fail(MK_ERR_UNSUPPORTED, "MK_MODE_MEGAKERNEL supports at most 256 query heads");
    if (cfg->flags & (MK_FLAG_FUSED_MERGE | MK_FLAG_NO_GRAPH | MK_FLAG_TILED_WEIGHTS | MK_FLAG_POISON))
      return fail(MK_ERR_INVALID_ARG, "FUSED_MERGE, NO_GRAPH, TILED_WEIGHTS and POISON are per-operator flags");
  }

  int dev_cus = 0, max_lds = 0;
  double tpu = 100.0;
  MK_TRY(device_facts(&dev_cus, &tpu, &max_lds));
  const int ncu = cfg->num_cus > 0 ? std::min(cfg->num_cus, dev_cus) : dev_cus;
  if (ncu < 1) return fail(MK_ERR_HIP, "no compute units reported");
  if (cfg->mode == MK_MODE_MEGAKERNEL && ncu > 256)
    return fail(MK_ERR_UNSUPPORTED, "MK_MODE_MEGAKERNEL runs on at most 256 compute units (set num_cus)");

  auto* h = new mk_handle();
  std::unique_ptr<mk_handle> guard(h);
  h->cfg = *cfg;
  h->stream = static_cast<hipStream_t>(hip_stream);
  HIP_TRY(hipGetDevice(&h->device));
  h->ticks_per_us = tpu;

  const GraphConfig gc = graph_config(cfg, ncu);
  h->batched = cfg->max_batch > 1;
  if (h->batched) {  // launches are issued per operator, stage by stage of the batched graph
    h->graph.cfg = gc;
    h->graph.nsplit = (cfg->max_seq + gc.split - 1) / gc.split;
    std::string e = build_batched_graph(batched_config(cfg, ncu, h->graph.nsplit), h->bgraph);
    if (!e.empty()) return fail(MK_ERR_INVALID_ARG, e);
    e = validate_batched_graph(h->bgraph);
    if (!e.empty()) return fail(MK_ERR_INVALID_ARG, "batched graph validation: " + e);
  } else {
    std::string e = build_graph(gc, h->graph);
    if (!e.empty()) return fail(MK_ERR_INVALID_ARG, e);
    e = validate_graph(h->graph);
    if (!e.empty()) return fail(MK_ERR_INVALID_ARG, "graph validation: " + e);
  }
  const Graph& g = h->graph;

  const int L = cfg->n_layers, H = cfg->hidden, nq = cfg->n_q_heads, nkv = cfg->n_kv_heads, hd = cfg->head_dim;
  const int F = cfg->ffn, V = cfg->vocab, B = cfg->max_batch, S = cfg->max_seq, G = nq / nkv;
  Params& P = h->P;
  P.L = L; P.H = H; P.nq = nq; P.nkv = nkv; P.hd = hd; P.F = F; P.V = V; P.B = B; P.max_seq = S;
  P.split = gc.split; P.nsplit = g.nsplit; P.tied = cfg->tie_embeddings ? 1 : 0; P.eps = cfg->rms_eps;
  P.kv_f32 = cfg->kv_fp32 ? 1 : 0;
  P.ncu = ncu;
  const double wd_ms = cfg->watchdog_ms ? cfg->watchdog_ms : 2000.0;
  P.timeout_ticks = (uint32_t)std::min(4.0e9, wd_ms * 1000.0 * tpu);
  // One wait iteration takes well over 20 ns (a sleep plus a memory read), so
  // this limit trips only if the wall clock stops advancing.
  P.spin_limit = (uint32_t)std::min(4.0e9, wd_ms * 1000.0 * 50.0);
  if (cfg->flags & MK_FLAG_SPIN_LIMIT_1) P.spin_limit = 1;
  P.shuffle_seed = 0;
  P.o_delay_ticks = (uint32_t)(kMegaOPrefetchDelayUs * tpu);
  if (cfg->flags & MK_FLAG_SHUFFLE) {  // splitmix64 of the caller's seed, made nonzero
    uint64_t z = (uint64_t)cfg->debug_seed + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    P.shuffle_seed = (uint32_t)(z ^ (z >> 31)) | 1u;
  }
  P.embed = static_cast<const uint16_t*>(w->embed);
  P.lm_head = static_cast<const uint16_t*>(w->lm_head);
  P.final_norm = static_cast<const uint16_t*>(w->final_norm);

  // layer pointer tables
  const void* const* lists[9] = {w->attn_norm, w->wq, w->wk, w->wv, w->wo, w->ffn_norm, w->w_gate, w->w_up, w->w_down};
  const uint16_t** d_ptrs = nullptr;
  MK_TRY(h->alloc(&d_ptrs, 9 * (int64_t)L));
  std::vector<const void*> hp(9 * (size_t)L);
  for (int i = 0; i < 9; ++i)
    for (int l = 0; l < L; ++l) hp[(size_t)i * L + l] = lists[i][l];
  HIP_TRY(hipMemcpy(d_ptrs, hp.data(), hp.size() * sizeof(void*), hipMemcpyHostToDevice));
  h->host_w = hp;
  P.attn_norm = d_ptrs + 0 * L; P.wq = d_ptrs + 1 * L; P.wk = d_ptrs + 2 * L; P.wv = d_ptrs + 3 * L;
  P.wo = d_ptrs + 4 * L; P.ffn_norm = d_ptrs + 5 * L; P.w_gate = d_ptrs + 6 * L; P.w_up = d_ptrs + 7 * L;
  P.w_down = d_ptrs + 8 * L;

  // KV cache
  const int64_t kv_elems = (int64_t)L * B * nkv * S * hd, kv_bytes = kv_elems * (P.kv_f32 ? 4 : 2);
  {
    uint8_t *kc = nullptr, *vc = nullptr;
    MK_TRY(h->alloc(&kc, kv_bytes));
    MK_TRY(h->alloc(&vc, kv_bytes));
    HIP_TRY(hipMemset(kc, 0, kv_bytes));
    HIP_TRY(hipMemset(vc, 0, kv_bytes));
    P.kcache = kc;
    P.vcache = vc;
  }

  // activations, one allocation
  const int64_t n_xs = (int64_t)(L + 1) * B * H, n_xmid = (int64_t)L * B * H, n_q = (int64_t)L * B * nq * hd;
  const int64_t n_part = (int64_t)L * B * nkv * g.nsplit * G * (hd + 2), n_aout = n_q, n_h = (int64_t)L * B * F;
  h->act_floats = n_xs + n_xmid + n_q + n_part + n_aout + n_h;
  MK_TRY(h->alloc(&h->act, h->act_floats));
  HIP_TRY(hipMemset(h->act, 0, h->act_floats * 4));
  P.xs = h->act;
  P.xmid = P.xs + n_xs;
  P.q = P.xmid + n_xmid;
  P.attn_part = P.q + n_q;
  P.attn_out = P.attn_part + n_part;
  P.h = P.attn_out + n_aout;
  MK_TRY(h->alloc(&P.lm_part, B));
  HIP_TRY(hipMemset(P.lm_part, 0, B * sizeof(unsigned long long)));
  MK_TRY(h->alloc(&P.attn_count, (int64_t)B * nkv));
  HIP_TRY(hipMemset(P.attn_count, 0, (size_t)B * nkv * 4));
  if (h->batched) {  // bf16 MFMA operands; rows B..Bp-1 are zero and never written
    const int bt = batch_tiles(B);
    P.Bp = 16 * bt;
    const int64_t n_ax = 2ll * P.Bp * H, n_ao = 2ll * P.Bp * nq * hd, n_ah = 2ll * P.Bp * F;  // hi + lo planes
    uint16_t* ops = nullptr;
    MK_TRY(h->alloc(&ops, n_ax + n_ao + n_ah));
    HIP_TRY(hipMemset(ops, 0, (n_ax + n_ao + n_ah) * 2));
    P.ax = ops;
    P.ao = ops + n_ax;
    P.ah = ops + n_ax + n_ao;
    int64_t n_part = 1;
    for (int t : {TT_QKV, TT_O, TT_GU, TT_DOWN, TT_LM}) {
      if (bgemm_lds(bt) > max_lds) return fail(MK_ERR_UNSUPPORTED, "batched projection LDS need exceeds the device");
      HIP_TRY(hipFuncSetAttribute(bgemm_kernel(t, bt, tiled_ops(h, t), bgemm_gpw(P, t)),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, bgemm_lds(bt)));
      const int ks = bgemm_splits(P, t, ncu);
      if (ks > 1) n_part = std::max<int64_t>(n_part, (int64_t)ks * bgemm_groups(P, t) * 2 * 16 * P.Bp);
    }
    MK_TRY(h->alloc(&P.bpart, n_part));
  }

  // RoPE angle tables, computed in double precision
  {
    const int half = hd / 2;
    std::vector<float> cs((size_t)S * half), sn((size_t)S * half);
    for (int p = 0; p < S; ++p)
      for (int i = 0; i < half; ++i) {
        const double a = (double)p * std::pow((double)cfg->rope_theta, -2.0 * i / hd);
        cs[(size_t)p * half + i] = (float)std::cos(a);
        sn[(size_t)p * half + i] = (float)std::sin(a);
      }
    float *dc = nullptr, *ds = nullptr;
    MK_TRY(h->alloc(&dc, (int64_t)S * half));
    MK_TRY(h->alloc(&ds, (int64_t)S * half));
    HIP_TRY(hipMemcpy(dc, cs.data(), cs.size() * 4, hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(ds, sn.data(), sn.size() * 4, hipMemcpyHostToDevice));
    P.rope_cos = dc;
    P.rope_sin = ds;
  }

  // task tables
  Task* d_flat = nullptr;
  int32_t* d_qoff = nullptr;
  MK_TRY(h->alloc(&d_flat, (int64_t)g.flat.size()));
  MK_TRY(h->alloc(&d_qoff, (int64_t)g.queue_off.size()));
  HIP_TRY(hipMemcpy(d_flat, g.flat.data(), g.flat.size() * sizeof(Task), hipMemcpyHostToDevice));
  HIP_TRY(hipMemcpy(d_qoff, g.queue_off.data(), g.queue_off.size() * 4, hipMemcpyHostToDevice));
  P.tasks = d_flat;
  P.queue_off = d_qoff;
  MK_TRY(h->alloc(&P.events, (int64_t)g.event_count.size()));
  HIP_TRY(hipMemset(P.events, 0, g.event_count.size() * 4));
  MK_TRY(h->alloc(&P.status, kStatusWords));
  HIP_TRY(hipMemset(P.status, 0, kStatusWords * 4));
  P.trace_op = -1;
  if (cfg->flags & MK_FLAG_TRACE) {
    MK_TRY(h->alloc(&P.trace, 2 * (int64_t)g.tasks.size()));
    HIP_TRY(hipMemset(P.trace, 0, 16 * g.tasks.size()));
    P.trace_cap = (int32_t)g.tasks.size();
  }
  MK_TRY(h->alloc(&h->d_tok_scratch, B));
  MK_TRY(h->alloc(&h->d_step, 1));

  if (cfg->mode == MK_MODE_MEGAKERNEL) {  // tagged hand-over buffers, zero (tag 0: never a step's epoch)
    const int64_t qkvw = (int64_t)(nq + 2 * nkv) * hd;
    const int64_t n_x = (int64_t)(L + 1) * H, n_xmid = (int64_t)L * H, n_qkv = (int64_t)L * qkvw;
    const int64_t n_rec = (int64_t)L * nkv * g.nsplit * G * (hd + 2), n_attn = (int64_t)L * nq * hd;
    const int64_t n_h = (int64_t)L * F, total = n_x + n_xmid + n_qkv + n_rec + n_attn + n_h + ncu + 1;
    uint64_t* t = nullptr;
    MK_TRY(h->alloc(&t, total));
    HIP_TRY(hipMemset(t, 0, total * 8));
    MegaBufs& M = h->mega;
    M.x = t;
    M.xmid = M.x + n_x;
    M.qkv = M.xmid + n_xmid;
    M.rec = M.qkv + n_qkv;
    M.attn = M.rec + n_rec;
    M.h = M.attn + n_attn;
    M.key = M.h + n_h;
    M.tok = M.key + ncu;
    HIP_TRY(hipHostMalloc(&h->host_abort, 64, hipHostMallocMapped | hipHostMallocCoherent));
    *h->host_abort = 0;
    HIP_TRY(hipHostGetDevicePointer(reinterpret_cast<void**>(&M.host_abort), h->host_abort, 0));
    if (cfg->flags & MK_FLAG_TRACE) {
      h->mega_trace_words = (int64_t)(4 * L + 1) * ncu * kMegaTraceSlots;
      MK_TRY(h->alloc(&M.trace, h->mega_trace_words));
      HIP_TRY(hipMemset(M.trace, 0, h->mega_trace_words * 8));
    }
    // every GEMV operator's tasks must fit the compute waves' result slots
    const int counts[5] = {(nq + nkv) * (hd / 2) + (nkv * hd + kRowsQkv - 1) / kRowsQkv, (H + kRowsO - 1) / kRowsO,
                           (F + kRowsGuPerMatrix - 1) / kRowsGuPerMatrix, (H + kRowsDown - 1) / kRowsDown,
                           (V + kRowsLm - 1) / kRowsLm};
    for (int c : counts)
      if ((c + ncu * kMegaCompute - 1) / (ncu * kMegaCompute) > 64)
        return fail(MK_ERR_UNSUPPORTED, "MK_MODE_MEGAKERNEL: an operator has more than 64 tasks per compute wave "
                                        "on this many CUs");
    h->mega_fn = mega_kernel(H, nq * hd, F, hd, P.kv_f32 != 0, G, (cfg->flags & MK_FLAG_SHUFFLE) != 0);
    if (!h->mega_fn) return fail(MK_ERR_UNSUPPORTED, "no megakernel instance for this shape");
  }
  if (!h->batched) {
    const std::string e = check_op_tasks(h->graph);
    if (!e.empty()) return fail(MK_ERR_INVALID_ARG, "internal: " + e);
  }
  for (int t = TT_QKV; t <= TT_ARGMAX && !h->batched; ++t) {  // single-sequence operator kernels
    if (t == TT_ATTN || t == TT_MERGE) continue;  // launched by their own kernels
    int pfl = 0;
    if (t == TT_QKV || t == TT_GU || t == TT_LM) pfl = H;
    else if (t == TT_O) pfl = nq * hd;
    else if (t == TT_DOWN) pfl = F;
    h->op_page[t] = round_up(pfl, 8);
    const int rows = t == TT_QKV ? TaskShape<TT_QKV>::R : t == TT_O ? TaskShape<TT_O>::R
                   : t == TT_GU ? TaskShape<TT_GU>::R : t == TT_DOWN ? TaskShape<TT_DOWN>::R
                   : t == TT_LM ? TaskShape<TT_LM>::R : 0;
    const int depth = t == TT_QKV ? TaskShape<TT_QKV>::D : t == TT_O ? TaskShape<TT_O>::D
                    : t == TT_GU ? TaskShape<TT_GU>::D : t == TT_DOWN ? TaskShape<TT_DOWN>::D
                    : t == TT_LM ? TaskShape<TT_LM>::D : 0;
    h->op_exact[t] = rows > 0 && pfl % 512 == 0 && (pfl / 512) % depth == 0;
    // per-wave scratch: attention state, or the results of the wave's GEMV tasks
    h->op_sf[t] = kMaxTasksPerWave * (rows + 1);  // results + task ids
    h->op_lds[t] = (int)sizeof(Lds) + h->op_page[t] * 4 + kWaves * h->op_sf[t] * 4;
    if (h->op_lds[t] > max_lds)
      return fail(MK_ERR_UNSUPPORTED, "operator LDS need exceeds " + std::to_string(max_lds));
    const void* fn = op_kernel(t, h->op_exact[t]);
    HIP_TRY(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, h->op_lds[t]));
    h->op_grid_cap[t] = kOpWgsPerCu * ncu;
  }
  h->attn_lds = (G * hd + kAttnWaves * G * (hd + 2)) * 4;  // queries, then the waves' records
  h->attn_full_lds = (G * hd + kAttnFullWaves * G * (hd + 2)) * 4;
  if (std::max(h->attn_lds, h->attn_full_lds) > max_lds)
    return fail(MK_ERR_UNSUPPORTED, "attention LDS need exceeds the device limit");
  HIP_TRY(hipFuncSetAttribute(attn_split_kernel(P.kv_f32, G),
                              hipFuncAttributeMaxDynamicSharedMemorySize, h->attn_lds));
  HIP_TRY(hipFuncSetAttribute(attn_full_kernel(P.kv_f32, G),
                              hipFuncAttributeMaxDynamicSharedMemorySize, h->attn_full_lds));
  if (cfg->mode == MK_MODE_MEGAKERNEL) {
    h->lds_mega = mega_lds_bytes(H, nq, nkv, hd, F, &h->page_floats);
    if (h->lds_mega > max_lds)
      return fail(MK_ERR_UNSUPPORTED,
                  "megakernel LDS need " + std::to_string(h->lds_mega) + " B exceeds " + std::to_string(max_lds));
    // keep one persistent workgroup per CU: ask for more than half the LDS
    if (h->lds_mega <= max_lds / 2) h->lds_mega = max_lds / 2 + 1024;
    HIP_TRY(hipFuncSetAttribute(h->mega_fn, hipFuncAttributeMaxDynamicSharedMemorySize, h->lds_mega));
    int nb = 0;
    HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, h->mega_fn, kMegaWaves * kWave, h->lds_mega));
    if (nb < 1) return fail(MK_ERR_UNSUPPORTED, "the megakernel does not fit on a CU");
  }
  if (cfg->flags & MK_FLAG_BATCHED_PREFILL) {
    if (cfg->flags & MK_FLAG_TILED_WEIGHTS)
      return fail(MK_ERR_UNSUPPORTED, "MK_FLAG_BATCHED_PREFILL needs row-major weights (not MK_FLAG_TILED_WEIGHTS)");
    const int qd = nq * hd, kd = nkv * hd;
    h->pf_cap = h->pf_rows = std::max(kPrefillRows, B);
    const int64_t wy = std::max<int64_t>({(int64_t)qd + 2 * kd, 2 * (int64_t)F, H});
    const int64_t wk = std::max<int64_t>({(int64_t)H, qd, F});
    MK_TRY(h->alloc(&h->pf_x, (int64_t)h->pf_cap * H));
    MK_TRY(h->alloc(&h->pf_y, (int64_t)h->pf_cap * wy));
    MK_TRY(h->alloc(&h->pf_ops, 2 * (int64_t)h->pf_cap * wk));
    MK_TRY(h->alloc(&h->pf_logits, 2 * (int64_t)B * V));
    HIP_TRY(pf_prepare(hd));
    if (rocblas_create_handle(&h->blas) != rocblas_status_success)
      return fail(MK_ERR_HIP, "rocblas_create_handle failed");
    if (rocblas_set_stream(h->blas, h->stream) != rocblas_status_success)
      return fail(MK_ERR_HIP, "rocblas_set_stream failed");
  }
  HIP_TRY(hipDeviceSynchronize());
  *out = guard.release();
  return MK_OK;
}

mk_status mk_decode_step(mk_handle* h, const int32_t* d_in, int32_t* d_out, float* d_logits) {
  g_err.clear();
  if (!h || !d_in || !d_out) return fail(MK_ERR_INVALID_ARG, "NULL handle or token pointer");
  if (h->poisoned) return fail(MK_ERR_STATE, "handle poisoned by an earlier in-kernel error");
  if (h->length >= h->cfg.max_seq) return fail(MK_ERR_CAPACITY, "KV cache full");
  if (h->batch == 0) h->batch = h->cfg.max_batch;
  Step S{};
  S.epoch = ++h->epoch;
  S.pos = h->length;
  S.tokens = d_in;
  S.tok_stride = 1;
  S.out = d_out;
  S.logits = d_logits;
  S.nsteps = 1;
  MK_TRY(launch_step(h, S));
  h->length++;
  return MK_OK;
}

mk_status mk_generate(mk_handle* h, const int32_t* d_in, int32_t n, int32_t* d_out, float* d_logits) {
  g_err.clear();
  if (!h || !d_in || !d_out) return fail(MK_ERR_INVALID_ARG, "NULL handle or token pointer");
  if (n < 1) return fail(MK_ERR_INVALID_ARG, "n_steps must be >= 1");
  if (h->cfg.max_batch != 1) return fail(MK_ERR_UNSUPPORTED, "mk_generate runs one sequence (max_batch 1)");
  if (h->poisoned) return fail(MK_ERR_STATE, "handle poisoned by an earlier in-kernel error");
  if ((int64_t)h->length + n > h->cfg.max_seq) return fail(MK_ERR_CAPACITY, "n_steps past the KV-cache capacity");
  if (h->batch == 0) h->batch = 1;
  if (h->cfg.mode == MK_MODE_MEGAKERNEL) {  // one launch for all n steps
    Step S{};
    S.epoch = h->epoch + 1;
    S.pos = h->length;
    S.tokens = d_in;
    S.tok_stride = 1;
    S.out = d_out;
    S.logits = d_logits;
    S.nsteps = n;
    S.tok_step = 0;  // step i > 0 takes step i - 1's greedy id
    S.out_step = 1;
    MK_TRY(launch_step(h, S));
    h->epoch += (uint32_t)n;
    h->length += n;
    return MK_OK;
  }
  for (int i = 0; i < n; ++i) {  // per operator: one step graph per step, ids fed back on the device
    Step S{};
    S.epoch = ++h->epoch;
    S.pos = h->length;
    S.tokens = i == 0 ? d_in : d_out + i - 1;
    S.tok_stride = 1;
    S.out = d_out + i;
    S.logits = i == n - 1 ? d_logits : nullptr;
    S.nsteps = 1;
    MK_TRY(launch_step(h, S));
    h->length++;
  }
  return MK_OK;
}

namespace {
// out[M][N] (row stride ldo, fp32) = X W^T for the bf16 weights W [N][K] and
// X = hi + lo, the operand planes pf_ops [2][M][K] (high parts, then low).
// rocBLAS is column-major: out^T = W X^T with W^T stored [K][N] (lda K) and
// X^T stored [K][rows] (ldb K).  Up to kPrefillStack rows (the weights'
// bytes bound the time) one GEMM runs over the 2M stacked rows, so the
// weights are read once, and the low part's rows are then added to the high
// part's (out needs 2M rows; with fold_to the sums go there instead);
// beyond that (the matrix cores bound it) a second GEMM accumulates the low
// part into out.  Either way out = fl(hi W^T + lo W^T).
mk_status pf_gemm(mk_handle* h, const uint16_t* W, int N, int K, int M, float* out, int ldo,
                  float* fold_to = nullptr, int ld_fold = 0) {
  const float one = 1.0f, zero = 0.0f;
  const uint16_t* hi = h->pf_ops;
  const uint16_t* lo = h->pf_ops + (int64_t)M * K;
  auto gemm = [&](const uint16_t* x, int rows, const float* beta) -> mk_status {
    const rocblas_status st = rocblas_gemm_ex(
        h->blas, rocblas_operation_transpose, rocblas_operation_none, N, rows, K, &one, W, rocblas_datatype_bf16_r,
        K, x, rocblas_datatype_bf16_r, K, beta, out, rocblas_datatype_f32_r, ldo, out, rocblas_datatype_f32_r, ldo,
        rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    if (st != rocblas_status_success) return fail(MK_ERR_HIP, std::string("rocblas_gemm_ex: ") + rocblas_status_to_string(st));
    return MK_OK;
  };
  if (M <= kPrefillStack) {
    MK_TRY(gemm(hi, 2 * M, &zero));
    HIP_TRY(pf_fold(h->stream, out, ldo, M, fold_to ? fold_to : out, fold_to ? ld_fold : ldo, M, N));
    return MK_OK;
  }
  MK_TRY(gemm(hi, M, &zero));
  MK_TRY(gemm(lo, M, &one));
  if (fold_to) HIP_TRY(pf_fold(h->stream, out, ldo, 0, fold_to, ld_fold, M, N));
  return MK_OK;
}

// The whole prompt of every sequence, in chunks of rows (sequence b, position
// p0 + i), row r = b c + i.  Per layer: RMSNorm (for layers after the first,
// with the previous down projection's residual add) -> Q, K, V GEMMs -> RoPE
// and KV append -> causal attention over the cache -> O GEMM -> residual add
// and RMSNorm -> gate and up GEMMs -> SwiGLU -> down GEMM; after the last
// layer of the last chunk the residual add, the final norm and the LM head run
// on each sequence's last position only, then the argmax.
mk_status prefill_batched(mk_handle* h, const int32_t* d_tokens, int B, int P, int32_t* d_next, float* d_logits) {
  const Params& Pp = h->P;
  const int L = Pp.L, H = Pp.H, qd = Pp.nq * Pp.hd, kd = Pp.nkv * Pp.hd, F = Pp.F, V = Pp.V, wq = qd + 2 * kd;
  const int cmax = std::max(1, h->pf_rows / B);
  hipStream_t s = h->stream;
  float *X = h->pf_x, *Y = h->pf_y;
  uint16_t* ops = h->pf_ops;
  auto W = [&](int table, int l) { return static_cast<const uint16_t*>(h->host_w[(size_t)table * L + l]); };
  for (int p0 = 0, c = 0; p0 < P; p0 += c) {
    c = std::min(cmax, P - p0);
    const int M = B * c;
    HIP_TRY(pf_embed(s, Pp, d_tokens, P, B, c, p0, X));
    for (int l = 0; l < L; ++l) {
      HIP_TRY(pf_add_norm_split(s, Pp, X, l ? Y : nullptr, H, W(0, l), M, 1, 0, ops, ops + (int64_t)M * H));
      MK_TRY(pf_gemm(h, W(1, l), qd, H, M, Y, wq));
      MK_TRY(pf_gemm(h, W(2, l), kd, H, M, Y + qd, wq));
      MK_TRY(pf_gemm(h, W(3, l), kd, H, M, Y + qd + kd, wq));
      HIP_TRY(pf_rope_kv(s, Pp, l, Y, wq, B, c, p0));
      HIP_TRY(pf_attention(s, Pp, l, Y, wq, B, c, p0, ops, ops + (int64_t)M * qd));
      MK_TRY(pf_gemm(h, W(4, l), H, qd, M, Y, H));
      HIP_TRY(pf_add_norm_split(s, Pp, X, Y, H, W(5, l), M, 1, 0, ops, ops + (int64_t)M * H));
      MK_TRY(pf_gemm(h, W(6, l), F, H, M, Y, 2 * F));
      MK_TRY(pf_gemm(h, W(7, l), F, H, M, Y + F, 2 * F));
      HIP_TRY(pf_swiglu_split(s, Pp, Y, M, ops, ops + (int64_t)M * F));
      MK_TRY(pf_gemm(h, W(8, l), H, F, M, Y, H));
    }
    if (p0 + c == P) {
      HIP_TRY(pf_add_norm_split(s, Pp, X, Y, H, Pp.final_norm, B, c, c - 1, ops, ops + (int64_t)B * H));
      float* lg = d_logits ? d_logits : h->pf_logits;
      MK_TRY(pf_gemm(h, Pp.tied ? Pp.embed : Pp.lm_head, V, H, B, h->pf_logits, V, lg, V));
      HIP_TRY(pf_argmax(s, Pp, lg, B, d_next));
    }
  }
  h->length = P;
  return MK_OK;
}
}  // namespace

mk_status mk_prefill(mk_handle* h, const int32_t* d_tokens, int32_t B, int32_t P, int32_t* d_next, float* d_logits) {
  g_err.clear();
  if (!h || !d_tokens || !d_next) return fail(MK_ERR_INVALID_ARG, "NULL handle or token pointer");
  if (h->poisoned) return fail(MK_ERR_STATE, "handle poisoned by an earlier in-kernel error");
  if (h->length != 0) return fail(MK_ERR_STATE, "prefill requires an empty cache (call mk_reset)");
  if (P < 1) return fail(MK_ERR_INVALID_ARG, "prefill length must be >= 1");
  if (B < 1 || B > h->cfg.max_batch) return fail(MK_ERR_CAPACITY, "batch outside [1, max_batch]");
  if (B != h->cfg.max_batch) return fail(MK_ERR_UNSUPPORTED, "batch must equal max_batch");
  if (P > h->cfg.max_seq) return fail(MK_ERR_CAPACITY, "prompt longer than max_seq");
  h->batch = B;
  if (h->cfg.flags & MK_FLAG_BATCHED_PREFILL) return prefill_batched(h, d_tokens, B, P, d_next, d_logits);
  if (h->cfg.mode == MK_MODE_MEGAKERNEL) {  // B == 1: the whole prompt in one launch
    Step S{};
    S.epoch = h->epoch + 1;
    S.pos = 0;
    S.tokens = d_tokens;
    S.tok_stride = P;
    S.out = d_next;  // every step writes it; the last step's id stays
    S.logits = d_logits;
    S.nsteps = P;
    S.tok_step = 1;
    S.out_step = 0;
    MK_TRY(launch_step(h, S));
    h->epoch += (uint32_t)P;
    h->length = P;
    return MK_OK;
  }
  for (int p = 0; p < P; ++p) {
    Step S{};
    S.epoch = ++h->epoch;
    S.pos = p;
    S.tokens = d_tokens + p;
    S.tok_stride = P;
    const bool last = p == P - 1;
    S.out = last ? d_next : h->d_tok_scratch;
    S.logits = last ? d_logits : nullptr;
    S.nsteps = 1;
    MK_TRY(launch_step(h, S));
    h->length++;
  }
  return MK_OK;
}

namespace {
// Waits for the handle's stream.  In megakernel mode a host watchdog runs
// beside the in-kernel limits: if the stream has not drained 10 s plus 100 ms
// per launch since the last wait, it raises the host-mapped abort word, which
// every in-kernel wait polls, and then waits for the kernels to end.
mk_status drain(mk_handle* h) {
  if (h->cfg.mode == MK_MODE_MEGAKERNEL && h->host_abort) {
    const double limit_ms = 10000.0 + 100.0 * h->pending;
    const auto t0 = std::chrono::steady_clock::now();
    for (;;) {
      const hipError_t e = hipStreamQuery(h->stream);
      if (e == hipSuccess) break;
      if (e != hipErrorNotReady) return fail(MK_ERR_HIP, std::string("hipStreamQuery: ") + hipGetErrorString(e));
      const double ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
      if (ms > limit_ms) {
        __atomic_store_n(h->host_abort, 1u, __ATOMIC_SEQ_CST);
        h->poisoned = true;
        HIP_TRY(hipStreamSynchronize(h->stream));
        h->pending = 0;
        return fail(MK_ERR_TIMEOUT, "host watchdog: the megakernel did not finish; aborted");
      }
      std::this_thread::sleep_for(std::chrono::microseconds(200));
    }
    h->pending = 0;
    return MK_OK;
  }
  HIP_TRY(hipStreamSynchronize(h->stream));
  return MK_OK;
}
}  // namespace

mk_status mk_read_status(mk_handle* h, uint32_t out[16]) {
  if (!h || !out) return fail(MK_ERR_INVALID_ARG, "NULL argument");
  MK_TRY(drain(h));
  HIP_TRY(hipMemcpy(out, h->P.status, kStatusWords * 4, hipMemcpyDeviceToHost));
  return MK_OK;
}

mk_status mk_synchronize(mk_handle* h) {
  g_err.clear();
  if (!h) return fail(MK_ERR_INVALID_ARG, "NULL handle");
  uint32_t st[kStatusWords];
  MK_TRY(mk_read_status(h, st));
  if (st[1] == ST_TIMEOUT) {
    h->poisoned = true;
    static const char* kinds[] = {"?", "input page", "compute completions", "stager rendezvous", "tagged input",
                                  "queries/keys/values", "attention records", "LM-head keys"};
    const uint32_t kind = st[4] & 0xFF;
    return fail(MK_ERR_TIMEOUT, std::string("in-kernel watchdog: workgroup ") + std::to_string(st[2]) + ", wave " +
                                    std::to_string(st[3]) + ", operator " + std::to_string(st[4] >> 8) +
                                    ", waiting for " + kinds[kind < 8 ? kind : 0] + ": have " + std::to_string(st[5]) +
                                    ", need " + std::to_string(st[6]));
  }
  if (st[1] == ST_LDS) {
    h->poisoned = true;
    return fail(MK_ERR_HIP, "the persistent kernel ran with less LDS than it requested");
  }
  if (st[1] == ST_NONFINITE) {
    h->poisoned = true;
    return fail(MK_ERR_STATE, "non-finite logits");
  }
  if (st[1] == ST_BADTOKEN) {
    h->poisoned = true;
    return fail(MK_ERR_INVALID_ARG, "a token id outside [0, vocab) was fed to the kernel (clamped)");
  }
  if (h->poisoned) return fail(MK_ERR_STATE, "handle poisoned");
  return MK_OK;
}

mk_status mk_reset(mk_handle* h) {
  g_err.clear();
  if (!h) return fail(MK_ERR_INVALID_ARG, "NULL handle");
  MK_TRY(drain(h));
  if (h->poisoned) return fail(MK_ERR_STATE, "handle poisoned; destroy and recreate it");
  HIP_TRY(hipMemset(h->P.events, 0, h->graph.event_count.size() * 4));
  HIP_TRY(hipMemset(h->P.lm_part, 0, h->cfg.max_batch * sizeof(unsigned long long)));
  HIP_TRY(hipMemset(h->P.attn_count, 0, (size_t)h->cfg.max_batch * h->P.nkv * 4));
  HIP_TRY(hipDeviceSynchronize());
  h->length = 0;
  h->batch = 0;
  // the epoch keeps counting: megakernel words tagged before the reset can
  // never carry a later step's epoch
  return MK_OK;
}

mk_status mk_kv_view(mk_handle* h, mk_kv_layout* out) {
  if (!h || !out) return fail(MK_ERR_INVALID_ARG, "NULL argument");
  const auto& P = h->P;
  out->k = P.kcache;
  out->v = P.vcache;
  out->stride_pos = P.hd;
  out->stride_head = (int64_t)P.max_seq * P.hd;
  out->stride_batch = (int64_t)P.nkv * out->stride_head;
  out->stride_layer = (int64_t)P.B * out->stride_batch;
  out->length = h->length;
  out->batch = h->batch;
  out->elem_bytes = P.kv_f32 ? 4 : 2;
  return MK_OK;
}

mk_status mk_kv_read(mk_handle* h, void* k_host, void* v_host, int64_t bytes) {
  g_err.clear();
  if (!h || !k_host || !v_host) return fail(MK_ERR_INVALID_ARG, "NULL argument");
  const auto& P = h->P;
  const int64_t need = (int64_t)P.L * P.B * P.nkv * P.max_seq * P.hd * (P.kv_f32 ? 4 : 2);
  if (bytes != need) return fail(MK_ERR_INVALID_ARG, "bytes must equal the cache size " + std::to_string(need));
  MK_TRY(drain(h));
  HIP_TRY(hipMemcpy(k_host, P.kcache, (size_t)bytes, hipMemcpyDeviceToHost));
  HIP_TRY(hipMemcpy(v_host, P.vcache, (size_t)bytes, hipMemcpyDeviceToHost));
  return MK_OK;
}

void mk_destroy(mk_handle* h) {
  if (!h) return;
  (void)drain(h);
  delete h;
}

// ---- debug / inspection ------------------------------------------------------

mk_status mk_graph_inspect(const mk_config* cfg, int32_t ncu, mk_graph_info* out) {
  g_err.clear();
  const std::string cerr = check_config(cfg);
  if (!cerr.empty()) return fail(MK_ERR_INVALID_ARG, cerr);
  if (ncu < 1 || !out) return fail(MK_ERR_INVALID_ARG, "ncu < 1 or out NULL");
  const GraphConfig gc = graph_config(cfg, ncu);
  if (cfg->max_batch > 1) {  // the batched launch plan: stages of tasks
    BatchedGraph bg;
    std::string e = build_batched_graph(batched_config(cfg, ncu, (cfg->max_seq + gc.split - 1) / gc.split), bg);
    if (!e.empty()) return fail(MK_ERR_INVALID_ARG, e);
    e = validate_batched_graph(bg);
    if (!e.empty()) return fail(MK_ERR_INVALID_ARG, "batched graph validation: " + e);
    *out = mk_graph_info{};
    out->n_tasks = (int32_t)bg.tasks.size();
    out->n_stages = (int32_t)bg.stages.size();
    out->ncu = ncu;
    out->nsplit = bg.cfg.nsplit;
    out->split = gc.split;
    out->min_queue = 1 << 30;
    for (const BStage& s : bg.stages) {  // per launch: workgroups (tasks) of the stage
      out->max_queue = std::max(out->max_queue, s.count);
      out->min_queue = std::min(out->min_queue, s.count);
    }
    out->weight_bytes = batched_weight_bytes(bg);
    return MK_OK;
  }
  Graph g;
  std::string e = build_graph(gc, g);
  if (!e.empty()) return fail(MK_ERR_INVALID_ARG, e);
  e = validate_graph(g);
  if (!e.empty()) return fail(MK_ERR_INVALID_ARG, "graph validation: " + e);
  e = check_op_tasks(g);
  if (!e.empty()) return fail(MK_ERR_INVALID_ARG, "internal: " + e);
  out->n_tasks = (int32_t)g.tasks.size();
  out->n_events = (int32_t)g.event_count.size();
  out->n_stages = (int32_t)g.stage_begin.size() - 1;
  out->ncu = ncu;
  out->nsplit = g.nsplit;
  out->split = gc.split;
  out->max_queue = 0;
  out->min_queue = 1 << 30;
  out->max_cu_bytes = 0;
  out->min_cu_bytes = INT64_MAX;
  out->weight_bytes = 0;
  for (int cu = 0; cu < ncu; ++cu) {
    const int n = (int)g.queues[cu].size();
    out->max_queue = std::max(out->max_queue, n);
    out->min_queue = std::min(out->min_queue, n);
    int64_t bytes = 0;
    for (int id : g.queues[cu]) bytes += task_weight_bytes(gc, g.tasks[id]);
    out->max_cu_bytes = std::max(out->max_cu_bytes, bytes);
    out->min_cu_bytes = std::min(out->min_cu_bytes, bytes);
    out->weight_bytes += bytes;
  }
  return MK_OK;
}

mk_status mk_batched_graph_fault(const mk_config* cfg, int32_t ncu, int32_t fault) {
  g_err.clear();
  const std::string cerr = check_config(cfg);
  if (!cerr.empty()) return fail(MK_ERR_INVALID_ARG, cerr);
  if (ncu < 1 || cfg->max_batch < 2) return fail(MK_ERR_INVALID_ARG, "ncu < 1 or max_batch < 2");
  const GraphConfig gc = graph_config(cfg, ncu);
  BatchedGraph g;
  std::string e = build_batched_graph(batched_config(cfg, ncu, (cfg->max_seq + gc.split - 1) / gc.split), g);
  if (!e.empty()) return fail(MK_ERR_INVALID_ARG, e);
  auto find = [&](uint8_t kind, int type, int from) {
    for (int s = from; s < (int)g.stages.size(); ++s)
      if (g.stages[s].kind == kind && (type < 0 || g.stages[s].type == type)) return s;
    return -1;
  };
  switch (fault) {
    case 1: {  // a projection workgroup computes its neighbour's row block
      int s = -1;
      for (int t : {TT_QKV, TT_O, TT_GU, TT_DOWN, TT_LM})
        if (s < 0 && g.cfg.gemm[t].blocks > 1) s = find(BK_GEMM, t, 0);
      if (s < 0) return fail(MK_ERR_UNSUPPORTED, "no projection with two row blocks");
      BTask& t = g.tasks[g.stages[s].first + 1];
      t.a0 = g.tasks[g.stages[s].first].a0;
      break;
    }
    case 2: {  // a finishing task takes its neighbour's row group
      const int s = find(BK_FIN, -1, 0);
      if (s < 0 || g.stages[s].count < 2) return fail(MK_ERR_UNSUPPORTED, "no split projection");
      g.tasks[g.stages[s].first + 1].a0 = g.tasks[g.stages[s].first].a0;
      break;
    }
    case 3: {  // the O projection runs before the attention output is complete
      const int so = find(BK_GEMM, TT_O, 0);
      if (so < 1) return fail(MK_ERR_UNSUPPORTED, "no O projection");
      const int sp = so - 1;  // the stage before it (the merge, or the attention itself)
      std::vector<BTask> moved;
      for (int i = g.stages[so].first; i < g.stages[so].first + g.stages[so].count; ++i) moved.push_back(g.tasks[i]);
      std::vector<BTask> prev(g.tasks.begin() + g.stages[sp].first,
                              g.tasks.begin() + g.stages[sp].first + g.stages[sp].count);
      const int first = g.stages[sp].first;
      for (auto& t : moved) t.stage = sp;
      for (auto& t : prev) t.stage = so;
      std::copy(moved.begin(), moved.end(), g.tasks.begin() + first);
      std::copy(prev.begin(), prev.end(), g.tasks.begin() + first + (int)moved.size());
      std::swap(g.stages[so], g.stages[sp]);
      g.stages[sp].first = first;
      g.stages[so].first = first + (int)moved.size();
      break;
    }
    case 4: {  // the down projection's finishing launch expects one more K split
      if (g.cfg.gemm[TT_DOWN].splits < 2) return fail(MK_ERR_UNSUPPORTED, "down projection not split");
      g.cfg.gemm[TT_DOWN].splits += 1;
      // the projection stages keep the workgroups that ran: re-derive only the finishing reads
      for (auto& s : g.stages)
        if (s.kind == BK_GEMM && s.type == TT_DOWN) s.gy = g.cfg.gemm[TT_DOWN].splits - 1;
      break;
    }
    case 5: {  // the last attention split of a KV head repeats the first
      const int s = find(BK_ATTN, -1, 0);
      if (s < 0 || g.cfg.nsplit < 2) return fail(MK_ERR_UNSUPPORTED, "attention not split");
      g.tasks[g.stages[s].first + g.cfg.nsplit - 1].a1 = 0;
      break;
    }
    default: return fail(MK_ERR_INVALID_ARG, "unknown fault");
  }
  e = validate_batched_graph(g);
  if (!e.empty()) return fail(MK_ERR_INVALID_ARG, "batched graph validation: " + e);
  return MK_OK;
}

mk_status mk_graph_simulate(const mk_config* cfg, int32_t ncu, uint64_t seed, int32_t workers, int32_t drop_event,
                            mk_sim_result* out) {
  g_err.clear();
  const std::string cerr = check_config(cfg);
  if (!cerr.empty()) return fail(MK_ERR_INVALID_ARG, cerr);
  if (ncu < 1 || !out || workers < 1 || workers > kWorkers) return fail(MK_ERR_INVALID_ARG, "bad ncu/workers/out");
  Graph g;
  std::string e = build_graph(graph_config(cfg, ncu), g);
  if (!e.empty()) return fail(MK_ERR_INVALID_ARG, e);
  SimResult r = simulate_graph(g, seed, workers, drop_event);
  out->completed = r.completed ? 1 : 0;
  out->executed = r.executed;
  out->blocked_event = r.blocked_event;
  out->race = r.error.empty() ? 0 : 1;
  if (!r.error.empty()) g_err = r.error;
  return MK_OK;
}

mk_status mk_graph_export(const mk_config* cfg, int32_t ncu, void* out, int32_t* cu, int32_t cap, int32_t* n) {
  g_err.clear();
  const std::string cerr = check_config(cfg);
  if (!cerr.empty()) return fail(MK_ERR_INVALID_ARG, cerr);
  if (ncu < 1 || !n) return fail(MK_ERR_INVALID_ARG, "ncu < 1 or n NULL");
  Graph g;
  std::string e = build_graph(graph_config(cfg, ncu), g);
  if (!e.empty()) return fail(MK_ERR_INVALID_ARG, e);
  *n = (int32_t)g.tasks.size();
  if ((out || cu) && cap < *n) return fail(MK_ERR_CAPACITY, "capacity too small");
  if (out) std::memcpy(out, g.tasks.data(), g.tasks.size() * sizeof(Task));
  if (cu) std::memcpy(cu, g.cu_of.data(), g.cu_of.size() * 4);
  return MK_OK;
}

mk_status mk_get_debug_view(mk_handle* h, mk_debug_view* out) {
  if (!h || !out) return fail(MK_ERR_INVALID_ARG, "NULL argument");
  out->xs = h->P.xs;
  out->xmid = h->P.xmid;
  out->q = h->P.q;
  out->attn_out = h->P.attn_out;
  out->h = h->P.h;
  out->events = h->P.events;
  out->n_events = (int32_t)h->graph.event_count.size();
  out->n_tasks = (int32_t)h->graph.tasks.size();
  out->ncu = h->P.ncu;
  out->nsplit = h->P.nsplit;
  out->split = h->P.split;
  out->lds_bytes = h->lds_mega;
  out->exact_ops = 0;
  for (int t = 0; t < 9; ++t) {
    if (h->op_exact[t]) out->exact_ops |= 1u << t;
    out->op_grid[t] = h->op_grid[t];
  }
  return MK_OK;
}

mk_status mk_time_ops(mk_handle* h, uint32_t type_mask, int32_t max_launches) {
  g_err.clear();
  if (!h || max_launches < 0) return fail(MK_ERR_INVALID_ARG, "bad arguments");
  if (h->cfg.mode != MK_MODE_PER_OP && type_mask) return fail(MK_ERR_UNSUPPORTED, "operator timing needs MK_MODE_PER_OP");
  HIP_TRY(hipStreamSynchronize(h->stream));
  const size_t need = 2 * (size_t)max_launches;
  while (h->ev_pool.size() < need) {
    hipEvent_t e;
    HIP_TRY(hipEventCreate(&e));
    h->ev_pool.push_back(e);
  }
  h->ev_type.assign(max_launches, 0);
  h->ev_used = 0;
  h->timed_mask = type_mask;
  return MK_OK;
}

mk_status mk_read_op_times(mk_handle* h, double* total_ms, int32_t* launches) {
  g_err.clear();
  if (!h || !total_ms || !launches) return fail(MK_ERR_INVALID_ARG, "NULL argument");
  HIP_TRY(hipStreamSynchronize(h->stream));
  for (int t = 0; t < 9; ++t) { total_ms[t] = 0; launches[t] = 0; }
  for (int i = 0; i < h->ev_used; ++i) {
    float ms = 0;
    HIP_TRY(hipEventElapsedTime(&ms, h->ev_pool[2 * i], h->ev_pool[2 * i + 1]));
    total_ms[h->ev_type[i]] += ms;
    launches[h->ev_type[i]] += 1;
  }
  h->ev_used = 0;
  h->timed_mask = 0;
  return MK_OK;
}

mk_status mk_time_op_replay(mk_handle* h, int32_t type, int32_t reps, double* total_ms, int32_t* launches) {
  g_err.clear();
  if (!h || !total_ms || !launches || reps < 1 || reps > 10000) return fail(MK_ERR_INVALID_ARG, "bad arguments");
  if (h->cfg.mode != MK_MODE_PER_OP) return fail(MK_ERR_UNSUPPORTED, "operator replay needs MK_MODE_PER_OP");
  // the LM head accumulates its argmax across launches and the argmax consumes
  // it: replaying either would change the next step's token
  if (type < 0 || type > TT_DOWN || (type == 0 && !h->batched))
    return fail(MK_ERR_INVALID_ARG, "replay supports the norm (batched path), QKV, attention, merge, O, gate/up "
                                    "and down launches");
  // the batched path's operand planes are shared by the layers: a replayed
  // QKV launch would append K/V computed from another layer's input
  if (h->batched && type == TT_QKV)
    return fail(MK_ERR_INVALID_ARG, "replay of the batched QKV launches would rewrite the KV cache");
  if (h->length < 1) return fail(MK_ERR_STATE, "replay needs a prefilled sequence");
  if (h->timed_mask) return fail(MK_ERR_STATE, "operator event timing is active");
  for (hipEvent_t& e : h->rep_ev)
    if (!e) HIP_TRY(hipEventCreate(&e));
  HIP_TRY(hipStreamSynchronize(h->stream));
  h->only_type = type;
  h->replayed = 0;
  mk_status st = MK_OK;
  if (hipEventRecord(h->rep_ev[0], h->stream) != hipSuccess) st = fail(MK_ERR_HIP, "hipEventRecord failed");
  for (int r = 0; r < reps && st == MK_OK; ++r) st = enqueue_ops(h, h->stream, false);
  h->only_type = -1;
  MK_TRY(st);
  HIP_TRY(hipEventRecord(h->rep_ev[1], h->stream));
  HIP_TRY(hipEventSynchronize(h->rep_ev[1]));
  float ms = 0;
  HIP_TRY(hipEventElapsedTime(&ms, h->rep_ev[0], h->rep_ev[1]));
  *total_ms = ms;
  *launches = h->replayed;
  return MK_OK;
}

mk_status mk_trace_op(mk_handle* h, int32_t type, int32_t layer) {
  g_err.clear();
  if (!h) return fail(MK_ERR_INVALID_ARG, "NULL handle");
  if (!h->P.trace) return fail(MK_ERR_STATE, "handle created without MK_FLAG_TRACE");
  if (!(h->cfg.flags & MK_FLAG_NO_GRAPH)) return fail(MK_ERR_STATE, "operator tracing needs MK_FLAG_NO_GRAPH");
  h->P.trace_op = type < 0 ? -1 : (type << 16) | layer;
  return MK_OK;
}

mk_status mk_mega_trace(mk_handle* h, uint64_t* out, int64_t cap, int32_t* ops, int32_t* ncu, int32_t* slots,
                        double* ticks_per_us) {
  g_err.clear();
  if (!h) return fail(MK_ERR_INVALID_ARG, "NULL handle");
  if (!h->mega.trace) return fail(MK_ERR_STATE, "megakernel handle created without MK_FLAG_TRACE");
  if (ops) *ops = 4 * h->P.L + 1;
  if (ncu) *ncu = h->P.ncu;
  if (slots) *slots = kMegaTraceSlots;
  if (ticks_per_us) *ticks_per_us = h->ticks_per_us;
  if (!out) return MK_OK;
  if (cap < h->mega_trace_words) return fail(MK_ERR_CAPACITY, "capacity too small");
  MK_TRY(drain(h));
  HIP_TRY(hipMemcpy(out, h->mega.trace, 8 * (size_t)h->mega_trace_words, hipMemcpyDeviceToHost));
  return MK_OK;
}

mk_status mk_get_mega_view(mk_handle* h, mk_mega_view* out) {
  if (!h || !out) return fail(MK_ERR_INVALID_ARG, "NULL argument");
  if (h->cfg.mode != MK_MODE_MEGAKERNEL) return fail(MK_ERR_STATE, "not a megakernel handle");
  out->x = h->mega.x;
  out->xmid = h->mega.xmid;
  out->qkv = h->mega.qkv;
  out->attn = h->mega.attn;
  out->h = h->mega.h;
  out->epoch = h->epoch;
  return MK_OK;
}

mk_status mk_t_stream_read(const void* src, int64_t bytes, int32_t wgs, int32_t loads, int32_t reps, void* stream,
                           float* best_ms) {
  g_err.clear();
  if (!src || !best_ms || bytes < 16 || bytes % 16 || wgs < 1 || reps < 1 || (loads != 4 && loads != 8 && loads != 16))
    return fail(MK_ERR_INVALID_ARG, "bad stream-read arguments");
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t* sink = nullptr;
  HIP_TRY(hipMalloc(&sink, 4));
  hipEvent_t e0, e1;
  HIP_TRY(hipEventCreate(&e0));
  HIP_TRY(hipEventCreate(&e1));
  float best = 1e30f;
  hipError_t err = hipSuccess;
  for (int r = 0; r < reps && err == hipSuccess; ++r) {
    err = hipEventRecord(e0, st);
    if (err == hipSuccess) err = launch_stream_read(src, bytes / 16, wgs, loads, sink, st);
    if (err == hipSuccess) err = hipEventRecord(e1, st);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    if (err == hipSuccess) best = std::min(best, ms);
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipFree(sink);
  if (err != hipSuccess) return fail(MK_ERR_HIP, std::string("stream read: ") + hipGetErrorString(err));
  *best_ms = best;
  return MK_OK;
}

mk_status mk_read_trace(mk_handle* h, uint64_t* out, int32_t cap, int32_t* n, double* ticks_per_us) {
  if (!h || !n) return fail(MK_ERR_INVALID_ARG, "NULL argument");
  if (!h->P.trace) return fail(MK_ERR_STATE, "handle created without MK_FLAG_TRACE");
  *n = h->P.trace_cap;
  if (ticks_per_us) *ticks_per_us = h->ticks_per_us;
  if (!out) return MK_OK;
  if (cap < h->P.trace_cap) return fail(MK_ERR_CAPACITY, "capacity too small");
  HIP_TRY(hipStreamSynchronize(h->stream));
  HIP_TRY(hipMemcpy(out, h->P.trace, 16 * (size_t)h->P.trace_cap, hipMemcpyDeviceToHost));
  return MK_OK;
}

// ---- single bodies -----------------------------------------------------------

mk_status mk_t_gemv(const void* W, const float* x, float* y, int32_t N, int32_t K, void* stream) {
  g_err.clear();
  if (!W || !x || !y || N < 1 || K < 8 || K % 8) return fail(MK_ERR_INVALID_ARG, "bad gemv arguments");
  int max_lds = 0;
  MK_TRY(device_facts(nullptr, nullptr, &max_lds));
  const int lds = K * 4;
  if (lds > max_lds) return fail(MK_ERR_UNSUPPORTED, "K too large for LDS staging");
  HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void*>(&mk_t_gemv_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds));
  const int grid = std::min((N + kWaves * 4 - 1) / (kWaves * 4), 1024);
  hipLaunchKernelGGL(mk_t_gemv_kernel, dim3(grid), dim3(kWaves * kWave), (unsigned)lds,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(W), x, y, N, K);
  HIP_TRY(hipGetLastError());
  return MK_OK;
}

mk_status mk_t_rmsnorm(const float* x, const void* gamma, float eps, float* y, int32_t n, void* stream) {
  g_err.clear();
  if (!x || !gamma || !y || n < 8 || n % 8) return fail(MK_ERR_INVALID_ARG, "bad rmsnorm arguments");
  int max_lds = 0;
  MK_TRY(device_facts(nullptr, nullptr, &max_lds));
  if (n * 4 > max_lds) return fail(MK_ERR_UNSUPPORTED, "n too large");
  HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void*>(&mk_t_rmsnorm_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, n * 4));
  hipLaunchKernelGGL(mk_t_rmsnorm_kernel, dim3(1), dim3(256), (unsigned)(n * 4), static_cast<hipStream_t>(stream), x,
                     static_cast<const uint16_t*>(gamma), eps, y, n);
  HIP_TRY(hipGetLastError());
  return MK_OK;
}

mk_status mk_t_attention(const float* q, const void* k, const void* v, int64_t head_stride, int32_t nq, int32_t nkv,
                         int32_t hd, int32_t T, int32_t split, int32_t kv_f32, float* o, void* stream) {
  g_err.clear();
  if (!q || !k || !v || !o || nq < 1 || nkv < 1 || nq % nkv || nq / nkv > kMaxGqa || (hd != 64 && hd != 128) ||
      T < 1 || split < 1 || split > kMaxSplit || head_stride < (int64_t)T * hd)
    return fail(MK_ERR_INVALID_ARG, "bad attention arguments");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int G = nq / nkv, nsplit = (T + split - 1) / split;
  float* part = nullptr;
  HIP_TRY(hipMalloc(&part, (size_t)nkv * nsplit * G * (hd + 2) * 4));
  const unsigned lds = (unsigned)((G * hd + G * kWave) * 4);
  const int f32 = kv_f32 ? 1 : 0;
  hipLaunchKernelGGL(mk_t_attn_partial_kernel, dim3(nkv * nsplit), dim3(kWave), lds, st, q, k, v, head_stride, nq,
                     nkv, hd, T, split, nsplit, f32, part);
  hipLaunchKernelGGL(mk_t_attn_merge_kernel, dim3(nkv), dim3(kWave), 0, st, part, nq, nkv, hd, T, split, nsplit, o);
  hipError_t e = hipStreamSynchronize(st);
  (void)hipFree(part);
  if (e != hipSuccess) return fail(MK_ERR_HIP, std::string("attention: ") + hipGetErrorString(e));
  return MK_OK;
}

// ---- allocation-free split-KV attention ------------------------------------
// The partial records of mk_t_attention_noalloc live in one file-scope device
// array.  On the host its name is only a stand-in for the symbol: its device
// address, which differs per GPU, comes from hipGetSymbolAddress on the first
// call on each device and is the only way host code refers to the array.
namespace {
constexpr int64_t kNoAllocFloats = int64_t(1) << 20;  // 4 MiB of split records per device
__device__ __align__(256) float scratch[kNoAllocFloats];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

mk_status scratch_for_current_device(float** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(MK_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MK_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MK_OK;
}
}  // namespace

mk_status mk_t_attention_noalloc(const float* q, const void* k, const void* v, int64_t head_stride, int32_t nq,
                                 int32_t nkv, int32_t hd, int32_t T, int32_t split, int32_t kv_f32, float* o,
                                 void* stream) {
  g_err.clear();
  if (!q || !k || !v || !o || nq < 1 || nkv < 1 || nq % nkv || nq / nkv > kMaxGqa || (hd != 64 && hd != 128) ||
      T < 1 || split < 1 || split > kMaxSplit || head_stride < (int64_t)T * hd)
    return fail(MK_ERR_INVALID_ARG, "bad attention arguments");
  const int G = nq / nkv, nsplit = (T + split - 1) / split;
  const int64_t need = (int64_t)nkv * nsplit * G * (hd + 2);
  if (need > kNoAllocFloats)
    return fail(MK_ERR_CAPACITY, "split records need " + std::to_string(need) + " floats, more than the " +
                                     std::to_string(kNoAllocFloats) + " of the static scratch (use a larger split)");
  float* part = nullptr;
  MK_TRY(scratch_for_current_device(&part));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned lds = (unsigned)((G * hd + G * kWave) * 4);
  const int f32 = kv_f32 ? 1 : 0;
  // every (group, split, head) record is written before the merge reads it,
  // so nothing left by an earlier call needs clearing
  hipLaunchKernelGGL(mk_t_attn_partial_kernel, dim3(nkv * nsplit), dim3(kWave), lds, st, q, k, v, head_stride, nq,
                     nkv, hd, T, split, nsplit, f32, part);
  hipLaunchKernelGGL(mk_t_attn_merge_kernel, dim3(nkv), dim3(kWave), 0, st, part, nq, nkv, hd, T, split, nsplit, o);
  HIP_TRY(hipGetLastError());
  return MK_OK;
}

mk_status mk_t_set_prefill_rows(mk_handle* h, int32_t rows) {
  g_err.clear();
  if (!h) return fail(MK_ERR_INVALID_ARG, "NULL handle");
  if (!(h->cfg.flags & MK_FLAG_BATCHED_PREFILL)) return fail(MK_ERR_STATE, "handle created without MK_FLAG_BATCHED_PREFILL");
  if (rows < h->cfg.max_batch || rows > h->pf_cap) return fail(MK_ERR_INVALID_ARG, "rows outside [max_batch, 4096]");
  h->pf_rows = rows;
  return MK_OK;
}

mk_status mk_t_op_raw(mk_handle* h, int32_t type, int32_t layer, const float* x, float* y) {
  g_err.clear();
  if (!h || !x || !y) return fail(MK_ERR_INVALID_ARG, "NULL argument");
  if (h->batched) return fail(MK_ERR_UNSUPPORTED, "single-sequence operator kernels only (max_batch 1)");
  if (type != TT_QKV && type != TT_O && type != TT_GU && type != TT_DOWN && type != TT_LM)
    return fail(MK_ERR_INVALID_ARG, "type must be 1 (QKV), 4 (O), 5 (gate/up), 6 (down) or 7 (LM head)");
  if (layer < 0 || layer >= h->P.L || (type == TT_LM && layer != 0))
    return fail(MK_ERR_INVALID_ARG, "layer out of range (the LM head takes layer 0)");
  Params P = h->P;
  P.raw_in = x;
  P.raw_out = y;
  P.trace_op = -1;
  return launch_op(h, P, type, type == TT_LM ? h->P.L : layer, h->stream);
}

mk_status mk_t_bgemm(const void* W, const void* A, float* Y, int32_t N, int32_t K, int32_t B, int32_t tiled,
                     void* stream) {
  g_err.clear();
  if (!W || !A || !Y || N < 1 || K < 8 || K % 8 || B < 1 || B > kMaxBatch)
    return fail(MK_ERR_INVALID_ARG, "bad bgemm arguments");
  if (tiled && (N % 16 || K % 32)) return fail(MK_ERR_INVALID_ARG, "tiled weights need N % 16 == 0 and K % 32 == 0");
  const int lds = b_lds_bytes(batch_tiles(B));
  // A device query first: as the first HIP call of a process,
  // hipFuncSetAttribute reports that no device exists.
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void*>(&mk_t_bgemm_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds));
  hipLaunchKernelGGL(mk_t_bgemm_kernel, dim3((N + 32 * kBgemmWaves - 1) / (32 * kBgemmWaves)),
                     dim3(kBgemmWaves * kWave), (unsigned)lds,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(W),
                     static_cast<const uint16_t*>(A), Y, N, K, B, tiled ? 1 : 0);
  HIP_TRY(hipGetLastError());
  return MK_OK;
}

mk_status mk_tile_weights(const void* src, void* dst, int64_t N, int64_t K, void* stream) {
  g_err.clear();
  if (!src || !dst || src == dst || N < 16 || K < 32 || N % 16 || K % 32)
    return fail(MK_ERR_INVALID_ARG, "tiling needs distinct buffers, N % 16 == 0 and K % 32 == 0");
  const int64_t nv = N * K / 8;
  const int grid = (int)std::min<int64_t>((nv + 255) / 256, 4096);
  hipLaunchKernelGGL(mk_tile_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), N, K);
  HIP_TRY(hipGetLastError());
  return MK_OK;
}

mk_status mk_t_argmax(const float* x, int32_t n, int32_t* out, void* stream) {
  g_err.clear();
  if (!x || !out || n < 1) return fail(MK_ERR_INVALID_ARG, "bad argmax arguments");
  hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned long long* slot = nullptr;
  HIP_TRY(hipMalloc(&slot, 8));
  HIP_TRY(hipMemsetAsync(slot, 0, 8, st));
  const int grid = std::min((n + 255) / 256, 256);
  hipLaunchKernelGGL(mk_t_argmax_kernel, dim3(grid), dim3(256), 0, st, x, n, slot);
  hipLaunchKernelGGL(mk_t_argmax_final, dim3(1), dim3(64), 0, st, slot, out);
  hipError_t e = hipStreamSynchronize(st);
  (void)hipFree(slot);
  if (e != hipSuccess) return fail(MK_ERR_HIP, std::string("argmax: ") + hipGetErrorString(e));
  return MK_OK;
}

}  // extern "C"
