// Host-side task-graph (tGraph) builder, validator and CPU simulator.
//
// The builder follows the compiler half of MPK ("Compilar LLM en un
// MegaKernel ...", section "Parte 1. Compilador"; "MPK: A Compiler and Runtime
// for Mega-Kernelizing Tensor Programs", section 2 "La Carte au Niveau SM"):
// every operator of the decode step is cut into tasks small enough for one
// wavefront, tasks are placed on per-CU queues, and producers are wired to
// consumers through counting events.  Because a decode step's graph is fully
// known before launch, all placement is ahead of time (the AOT case of the MPK
// explainer's section 3).
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "mk_internal.h"

namespace mk {

struct GraphConfig {
  int L, H, nq, nkv, hd, F, V, B, max_seq, split, ncu;
};

struct Graph {
  GraphConfig cfg;
  int nsplit = 0;
  std::vector<Task> tasks;                 // by global id (topological order)
  std::vector<int> stage_of;               // stage index of each task
  std::vector<int> cu_of;                  // CU of each task
  std::vector<std::vector<int>> queues;    // per CU: task ids in execution order
  std::vector<uint32_t> event_count;       // signals per step of each event
  std::vector<int> stage_begin;            // tasks [stage_begin[s], stage_begin[s+1]) form stage s
  std::vector<uint8_t> stage_type;
  // device tables
  std::vector<Task> flat;                  // queue order, CU-major
  std::vector<int32_t> queue_off;          // [ncu + 1]
};

// Positions per split-KV attention task for a given max context.
int auto_split(int max_seq);

// Build the decode-step graph.  Returns "" on success, else a message.
std::string build_graph(const GraphConfig& cfg, Graph& g);

// Static checks: every task once; queues in topological order; event counts
// equal the number of signals; every output element written exactly once per
// step; every element a task (or its staged input) reads is written by a task
// the reader transitively waits for; RoPE pairs inside one task.
std::string validate_graph(const Graph& g);

struct SimResult {
  bool completed = false;
  int blocked_event = -1;   // an event some blocked task waits on
  int executed = 0;
  std::string error;        // race or protocol error, "" if none
};

// Run the per-CU queues under the runtime's protocol (scheduler frontier,
// worker tickets, staged pages, aggregated signals, event thresholds) in a
// random interleaving.  `drop_event` >= 0 suppresses one signal of that event
// (fault injection: the run must then report a deadlock on it).
SimResult simulate_graph(const Graph& g, uint64_t seed, int workers, int drop_event);

// ---------------------------------------------------------------------------
// Batched decode step (B >= 2 sequences).  Every operator runs on the matrix
// cores as launches of its own, so the task graph is a sequence of stages: a
// stage's tasks read only what earlier stages wrote (stream order is the
// dependency), and each stage is one launch whose grid is the stage's task
// grid.  The tiling comes from the same helpers the launches use; the graph
// is built and validated at create, and the step's launches are issued from
// it.
enum BKind : uint8_t { BK_NORM = 1, BK_GEMM, BK_FIN, BK_ATTN, BK_ATTN_FULL, BK_MERGE, BK_ARGMAX };

struct BGemm {     // tiling of one batched projection
  int groups;      // row groups: two 16-row tiles (gate/up: the same 16 rows of both matrices)
  int per_block;   // row groups per workgroup
  int blocks;      // workgroups along the rows
  int splits;      // workgroups along K (1: the epilogue runs in the projection launch)
  int chunk_cols;  // K columns per activation chunk
  int K, N;        // contraction length, output rows
};

struct BatchedConfig {
  int L, H, nq, nkv, hd, F, V, B, nsplit;
  bool fused_merge;  // the last split workgroup of each (sequence, KV head) merges (no merge launch)
  BGemm gemm[9];     // by operator type (TT_QKV, TT_O, TT_GU, TT_DOWN, TT_LM)
};

struct BTask {
  int stage;
  uint8_t kind, type;  // BK_*, operator type of GEMM / FIN tasks
  int layer, b;        // b: sequence (-1: every sequence)
  int a0, a1;          // GEMM: row block, K split; FIN: row group; ATTN: KV head, split; MERGE: KV head;
                       // NORM: 0 attention, 1 FFN, 2 final
};

struct BStage {
  uint8_t kind, type;
  int layer, sub;   // sub: NORM kind
  int first, count; // tasks [first, first + count)
  int gx, gy;       // launch grid in workgroups (0 x 0: done inside the previous launch)
};

struct BatchedGraph {
  BatchedConfig cfg;
  std::vector<BTask> tasks;
  std::vector<BStage> stages;
};

std::string build_batched_graph(const BatchedConfig& cfg, BatchedGraph& g);

// Every projection's (row group, K chunk) pairs covered once; every output
// element (per sequence) written exactly once per step; every split partial
// written once and read by its finishing task; every element a task reads
// written by an earlier stage.
std::string validate_batched_graph(const BatchedGraph& g);

// Weight bytes the GEMM tasks of the graph stream (bf16), for checking that
// the tiling reads every weight once.
int64_t batched_weight_bytes(const BatchedGraph& g);

}  // namespace mk
