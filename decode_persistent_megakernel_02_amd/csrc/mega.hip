// The persistent decode megakernel: one launch runs a whole decode step (every
// layer, the LM head and the argmax) with one workgroup resident on each CU.
//
// Method: the operator graph of the step is cut into tasks that each run on
// one compute unit, and a task runs as soon as the data it needs exists
// ("Compilar LLM en un MegaKernel ...", sections "Parte 1. Compilador" and
// "Parte 2. Runtime"; "MPK: A Compiler and Runtime for Mega-Kernelizing Tensor
// Programs", sections 2-4).  The pages' runtime signals events through counters
// in global memory.  On this device a counter event needs an agent-scope
// release before the increment and an acquire after the wait, and the two
// fences write back and invalidate the die's L2.  Measured with 256
// workgroups: a counter barrier takes 4 us, and 10 us with the fences.
// Here the dependency is carried by the data itself instead.  Every value one
// workgroup hands to another is a 64-bit word: the fp32 value in the low half
// and the step's epoch in the high half.  It is written and read with
// agent-scope relaxed atomics, which are coherent across the dies' L2s
// without fences.  A consumer re-reads a word until its tag equals the
// current epoch, so the tag is the event and no counter or fence is needed.
//
// A workgroup has kMegaStagers + kMegaCompute waves with fixed roles:
//  * stager waves (the pages' schedulers) wait for each operator's input
//    words, normalise the input (RMSNorm) into one of two LDS pages, and
//    publish the page to the compute waves through an LDS word.  Between the
//    QKV and O operators they also run the decode-attention units (one wave
//    per (KV head, split)), the log-sum-exp merges (one wave per query head)
//    and, at the end, the argmax.
//  * compute waves (the workers) stream the weight rows of their tasks: the
//    same GEMV bodies, rows per task and task order as the per-operator
//    kernels.  Weights depend on nothing, so a compute wave issues the loads
//    of its first two tasks of the next operator as soon as it has finished
//    the current one.  Those loads are in flight while the input is still
//    being produced elsewhere, and the weight stream does not stop at
//    operator boundaries.
// The roles keep activation loads and weight loads on different waves.  Vector
// loads of one wave complete in order, so a staging load queued behind a
// weight prefetch would wait for all of it.
//
// Every wait is bounded by a clock limit and an iteration limit.  Each wait
// also polls an LDS abort word, the device status word and a host-mapped
// abort word.  Waves coordinate only through LDS words and tagged global
// words: after the start-up barrier no wave waits at a workgroup barrier, so
// a wave that gives up can never strand the others.
#include "device.h"
#include "kernels.h"

namespace mk {

namespace {

constexpr int NS = kMegaStagers, NC = kMegaCompute;
constexpr int kR = TaskShape<TT_GU>::R, kD = TaskShape<TT_GU>::D;
static_assert(TaskShape<TT_QKV>::R == kR && TaskShape<TT_O>::R == kR && TaskShape<TT_DOWN>::R == kR &&
                  TaskShape<TT_LM>::R == kR,
              "the megakernel carries one weight-buffer shape across operators");
static_assert(TaskShape<TT_QKV>::D == kD && TaskShape<TT_O>::D == kD && TaskShape<TT_DOWN>::D == kD &&
                  TaskShape<TT_LM>::D == kD,
              "the megakernel carries one weight-buffer shape across operators");
constexpr int NB = 2;   // weight buffers (tasks in flight) per compute wave
// A compute wave holds at most kMegaMaxTasks results of one operator (lane j
// of pass p runs the epilogue of task 64 p + j).
constexpr int kMegaMaxTasks = 128;
// trace words per (operator, workgroup): compute waves' (duration, end), then
// the stager's publish time, poll start and input-complete time
constexpr int kTraceSlots = kMegaTraceSlots;

// ---- tagged words ----------------------------------------------------------
__device__ __forceinline__ void tput(uint64_t* p, float v, uint32_t epoch) {
  __hip_atomic_store(p, ((uint64_t)epoch << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tget(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tcur(uint64_t w, uint32_t epoch) { return (uint32_t)(w >> 32) == epoch; }
__device__ __forceinline__ float tval(uint64_t w) { return __uint_as_float((uint32_t)w); }

// LM-head key of a workgroup: ordered value (bits 63..32), 0x1FFFF - index
// (bits 31..15, so that larger means a smaller index), epoch mod 2^15.
__device__ __forceinline__ uint64_t key_pack(unsigned long long k, uint32_t epoch) {
  const uint32_t idx = 0xFFFFFFFFu - (uint32_t)k;  // k == 0 (no rows): index field 0, never the maximum
  return ((k >> 32) << 32) | ((uint64_t)((0x1FFFFu - idx) & 0x1FFFFu) << 15) | (epoch & 0x7FFFu);
}

__device__ __forceinline__ uint32_t lds_acq(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_rel_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_rel_add(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ---- bounded waits ----------------------------------------------------------
// s_sleep between re-reads of stale tagged words (64 clocks per unit): each
// round reads the stale words again from the memory-side caches.
#ifndef MK_POLL_SLEEP
#define MK_POLL_SLEEP 2
#endif
constexpr int kPollSleep = MK_POLL_SLEEP;
// One wait: tick() sleeps briefly and returns false when the wave must stop
// (abort raised anywhere, or this wait ran out of time or iterations; then it
// latches the timeout and raises the abort itself).
struct Spin {
  uint64_t t0;
  uint32_t it;
  // The clock is first read on the first unsuccessful check: a wait that is
  // already satisfied costs no clock read (s_memrealtime is a memory-path
  // instruction with a round trip of its own).
  __device__ __forceinline__ Spin() : t0(0), it(0) {}
  // sleep: s_sleep argument between checks (64 clocks each).  The device
  // status word and the host-mapped abort word are read only every 4096
  // checks: 2048 waiting waves reading host memory every few microseconds
  // would flood the fabric that the weight stream uses.
  template <int SLEEP = 2>
  __device__ __forceinline__ bool tick(const Params& P, const MegaBufs& M, MegaLds* L, uint32_t who, uint32_t what,
                                       uint32_t have, uint32_t need, int lane) {
    if (it++ == 0) t0 = clock_now();
    if (lds_load(&L->abort)) return false;
    if ((it & 4095) == 0) {
      if (__hip_atomic_load(&P.status[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ||
          __hip_atomic_load(M.host_abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)) {
        if (lane == 0) lds_store(&L->abort, 1u);
        return false;
      }
    }
    if (it > P.spin_limit || ((it & 63) == 0 && clock_now() - t0 > P.timeout_ticks)) {
      if (lane == 0) {
        if (atomicCAS(&P.status[1], ST_OK, ST_TIMEOUT) == ST_OK) {
          P.status[2] = blockIdx.x;
          P.status[3] = who;   // wave index in the workgroup
          P.status[4] = what;  // (op index << 8) | wait kind
          P.status[5] = have;
          P.status[6] = need;
          P.status[7] = 3;     // megakernel wait
        }
        __hip_atomic_store(&P.status[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lds_store(&L->abort, 1u);
      }
      return false;
    }
    __builtin_amdgcn_s_sleep(SLEEP);
    return true;
  }
};

// Wait kinds (low byte of `what`).
enum : uint32_t { W_READY = 1, W_DONE = 2, W_SYNC = 3, W_DATA = 4, W_QKV = 5, W_REC = 6, W_KEY = 7 };

// Waits until the LDS word reaches `need` (acquire).
__device__ __forceinline__ bool wait_lds(const Params& P, const MegaBufs& M, MegaLds* L, const uint32_t* w,
                                         uint32_t need, uint32_t who, uint32_t what, int lane) {
  Spin sp;
  uint32_t v;
  while ((v = lds_acq(w)) < need)
    if (!sp.tick(P, M, L, who, what, v, need, lane)) return false;
  return true;
}

// ---- the step's operator sequence ---------------------------------------------
// GEMV operators in order: per layer QKV (k = 4l), O, GU, DOWN; then the LM
// head (k = 4L).  Operator k stages its input into page k & 1.
__device__ __forceinline__ int op_type(int k, int L) {
  if (k == 4 * L) return TT_LM;
  const int m = k & 3;
  return m == 0 ? TT_QKV : m == 1 ? TT_O : m == 2 ? TT_GU : TT_DOWN;
}
__device__ __forceinline__ int op_count(const Params& P, int type) {
  switch (type) {
    case TT_QKV: return (P.nq + P.nkv) * (P.hd / 2) + (P.nkv * P.hd + kRowsQkv - 1) / kRowsQkv;
    case TT_O: return (P.H + kRowsO - 1) / kRowsO;
    case TT_GU: return (P.F + kRowsGuPerMatrix - 1) / kRowsGuPerMatrix;
    case TT_DOWN: return (P.H + kRowsDown - 1) / kRowsDown;
    default: return (P.V + kRowsLm - 1) / kRowsLm;
  }
}
// Compute-wave completions of page (k & 1) once operator k is done everywhere in this workgroup.
__device__ __forceinline__ uint32_t done_after(int k) { return (uint32_t)NC * (uint32_t)(k / 2 + 1); }
// ... and the count at which page (k & 1) is free for operator k (operator k - 2 done).
__device__ __forceinline__ uint32_t free_for(int k) { return (uint32_t)NC * (uint32_t)(k / 2); }

// ---- compute waves -------------------------------------------------------------
// Pool slot p of this workgroup's share of an operator's `count` tasks, or
// `count` past its end.  Workgroup b runs on die b % kXcds; the workgroups of
// one die share one contiguous part of the tasks and take them in turn, one
// task at a time, so every workgroup of a die gets the same number of tasks
// to within one (in runs of several tasks, an operator with 1.5 runs per
// workgroup -- QKV at the 8B shape -- gave half the workgroups twice the
// tasks of the others).
// rot (0 <= rot < count) rotates the task list: slot p then runs task
// (t + rot) mod count instead of t (MK_FLAG_SHUFFLE; 0 otherwise).
__device__ __forceinline__ int mslot_plain(uint32_t p, int count) {
  const int n = gridDim.x;
  if (n % kXcds) {
    const int t = (int)p * n + (int)blockIdx.x;
    return t < count ? t : count;
  }
  const int per = (count + kXcds - 1) / kXcds, x = (int)blockIdx.x % kXcds, j = (int)blockIdx.x / kXcds;
  const int t = (int)p * (n / kXcds) + j;
  return t < per && x * per + t < count ? x * per + t : count;
}
__device__ __forceinline__ int mslot(uint32_t p, int count, int rot) {
  int t = mslot_plain(p, count);
  if (rot == 0 || t >= count) return t;
  t += rot;
  return t < count ? t : t - count;
}

// The rotation of operator k's task list in the step with this epoch: 0, or
// in the shuffling instances (SHUF, MK_FLAG_SHUFFLE) a hash of (seed, epoch,
// k) reduced mod count (the 32-bit "lowbias32" integer mixer published by C.
// Wellons).  The production instances are compiled without it.
template <bool SHUF>
__device__ __forceinline__ int op_rot(const Params& P, int k, uint32_t epoch, int count) {
  if constexpr (!SHUF) return 0;
  if (!P.shuffle_seed) return 0;
  uint32_t h = P.shuffle_seed ^ (epoch * 0x9E3779B9u) ^ ((uint32_t)k * 0x85EBCA6Bu);
  h ^= h >> 16;
  h *= 0x7FEB352Du;
  h ^= h >> 15;
  h *= 0x846CA68Bu;
  h ^= h >> 16;
  return (int)(h % (uint32_t)count);
}

struct WBuf {
  v4u w[kD][kR];
  GemvRows<kR> g;
};

// Rows of task t of operator (type, layer): the per-operator kernels' task formula.
template <int TT>
__device__ __forceinline__ void setup_task(const Params& P, int layer, int t, GemvRows<kR>& g) {
  const Task d = op_task_fields(TT, layer, t, P.H, P.nq, P.nkv, P.hd, P.F, P.V, P.L);
  const uint16_t *W0, *W1 = nullptr;
  if constexpr (TT == TT_QKV) W0 = d.a0 == 0 ? ld_const(P.wq + layer) : d.a0 == 1 ? ld_const(P.wk + layer) : ld_const(P.wv + layer);
  else if constexpr (TT == TT_GU) { W0 = ld_const(P.w_gate + layer); W1 = ld_const(P.w_up + layer); }
  else if constexpr (TT == TT_O) W0 = ld_const(P.wo + layer);
  else if constexpr (TT == TT_DOWN) W0 = ld_const(P.w_down + layer);
  else W0 = P.tied ? P.embed : P.lm_head;
  gemv_setup_w<TT>(P, d, W0, W1, g);
}

template <int TT, bool EXACT>
__device__ __forceinline__ void fetch_task(const Params& P, int layer, int t, WBuf& b, int lane) {
  setup_task<TT>(P, layer, t, b.g);
  gemv_prefetch<kR, kD, EXACT>(b.w, b.g, lane);
}

// The first NB tasks of operator k for compute wave c: pool slots c, NC + c,
// 2 NC + c, ... (increasing, so the valid ones are a prefix).
template <int TT, bool EXACT>
__device__ __forceinline__ void fetch_first_t(const Params& P, int layer, int count, int rot, int c, WBuf (&B)[NB],
                                              int (&t)[NB], int lane) {
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    t[i] = mslot(i * NC + c, count, rot);
    if (t[i] < count) fetch_task<TT, EXACT>(P, layer, t[i], B[i], lane);
  }
}
// (epoch: the step operator k belongs to)
template <bool EXACT, bool SHUF>
__device__ __forceinline__ void fetch_first(const Params& P, int k, uint32_t epoch, int c, WBuf (&B)[NB],
                                            int (&t)[NB], int lane) {
  const int type = op_type(k, P.L), layer = type == TT_LM ? P.L : k / 4, count = op_count(P, type);
  const int rot = op_rot<SHUF>(P, k, epoch, count);
  switch (type) {
    case TT_QKV: fetch_first_t<TT_QKV, EXACT>(P, layer, count, rot, c, B, t, lane); break;
    case TT_O: fetch_first_t<TT_O, EXACT>(P, layer, count, rot, c, B, t, lane); break;
    case TT_GU: fetch_first_t<TT_GU, EXACT>(P, layer, count, rot, c, B, t, lane); break;
    case TT_DOWN: fetch_first_t<TT_DOWN, EXACT>(P, layer, count, rot, c, B, t, lane); break;
    default: fetch_first_t<TT_LM, EXACT>(P, layer, count, rot, c, B, t, lane); break;
  }
}

// Next pool slot's task, or `count` when the pool is empty or the wave's
// result slots would overflow (j results kept, NB - 1 tasks in flight).
__device__ __forceinline__ int mnext(uint32_t* pool, int j, int count, int rot, int lane) {
  if (j + NB > kMegaMaxTasks) return count;
  uint32_t p = 0;
  if (lane == 0) p = lds_add(pool, 1u);
  p = __builtin_amdgcn_readfirstlane(p);
  return mslot(p, count, rot);
}

// Streams the wave's tasks of one operator.  On entry buffer i holds task t[i]
// (in flight); each consumed buffer is refilled with the pool's next task.
// Every exit has its own unrolled drain, so the loads in flight at each
// consume are a fixed count.  Results go to res/ids; returns their number.
template <int TT, bool EXACT>
__device__ __forceinline__ int stream_op(const Params& P, int layer, int count, int rot, WBuf (&B)[NB],
                                         int (&t)[NB], const float* page, float* res, int* ids, uint32_t* pool,
                                         int lane) {
  float y[kR];
  int j = 0;
  if (t[NB - 1] >= count) {  // fewer than NB tasks: the valid prefix
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (t[i] < count) {
        gemv_run<kR, kD, EXACT>(B[i].w, B[i].g, page, lane, y);
        gemv_put<TT>(res, ids, j++, t[i], y, lane);
      }
    return j;
  }
  for (;;) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      gemv_run<kR, kD, EXACT>(B[i].w, B[i].g, page, lane, y);
      gemv_put<TT>(res, ids, j++, t[i], y, lane);
      const int n = mnext(pool, j, count, rot, lane);
      if (n >= count) {
#pragma unroll
        for (int m = 1; m < NB; ++m) {
          gemv_run<kR, kD, EXACT>(B[(i + m) % NB].w, B[(i + m) % NB].g, page, lane, y);
          gemv_put<TT>(res, ids, j++, t[(i + m) % NB], y, lane);
        }
        return j;
      }
      t[i] = n;
      fetch_task<TT, EXACT>(P, layer, n, B[i], lane);
    }
  }
}

// Epilogues of the wave's n tasks (lane j finishes task j), writing tagged words.
template <int TT>
__device__ __forceinline__ void finish_op(const Params& P, const MegaBufs& M, const Step& S, int layer, int n,
                                          const float* res, const int* ids, const float* resid, const float* rope,
                                          MegaLds* L, int lane) {
  __builtin_amdgcn_wave_barrier();
  const uint32_t ep = S.epoch;
  unsigned long long best = 0;
  // RMSNorm: the page holds gain * x, the stagers' sums of x^2 are in L->red;
  // the 1/rms factor is common to every row, so it scales the outputs
  float sc = 1.0f;
  if constexpr (TT == TT_QKV || TT == TT_GU || TT == TT_LM) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NS; ++w) tot += L->red[w];
    sc = 1.0f / sqrtf(tot / (float)P.H + P.eps);
  }
  for (int jj = lane; jj < n; jj += kWave) {
    const Task d = op_task_fields(TT, layer, ids[jj], P.H, P.nq, P.nkv, P.hd, P.F, P.V, P.L);
    float y[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) y[r] = res[jj * kR + r] * sc;
    if constexpr (TT == TT_QKV) {
      const int qd = P.nq * P.hd, kd = P.nkv * P.hd;
      uint64_t* out = M.qkv + (size_t)layer * (qd + 2 * kd);
      if (d.a3) {  // RoPE pair (a1, a1 + hd/2) of query (a0 = 0) or key (a0 = 1) rows
        const int half = P.hd / 2, i = d.a1 % P.hd;
        const float c = rope[i], sn = rope[half + i];
        const float lo = y[0] * c - y[1] * sn, hi = y[1] * c + y[0] * sn;
        uint64_t* o = out + (d.a0 == 0 ? 0 : qd);
        tput(o + d.a1, lo, ep);
        tput(o + d.a1 + d.a3, hi, ep);
      } else {
#pragma unroll
        for (int r = 0; r < kR; ++r)
          if (r < d.a2) tput(out + qd + kd + d.a1 + r, y[r], ep);
      }
    } else if constexpr (TT == TT_O) {
#pragma unroll
      for (int r = 0; r < kR; ++r)
        if (r < d.a2) tput(M.xmid + (size_t)layer * P.H + d.a1 + r, resid[d.a1 + r] + y[r], ep);
    } else if constexpr (TT == TT_GU) {
#pragma unroll
      for (int r = 0; r < kR / 2; ++r)
        if (r < d.a2) tput(M.h + (size_t)layer * P.F + d.a1 + r, silu(y[r]) * y[r + kR / 2], ep);
    } else if constexpr (TT == TT_DOWN) {
#pragma unroll
      for (int r = 0; r < kR; ++r)
        if (r < d.a2) tput(M.x + (size_t)(layer + 1) * P.H + d.a1 + r, resid[d.a1 + r] + y[r], ep);
    } else {
#pragma unroll
      for (int r = 0; r < kR; ++r)
        if (r < d.a2) {
          const int row = d.a1 + r;
          if (S.logits) S.logits[row] = y[r];
          const unsigned long long k = argmax_key(y[r], (uint32_t)row);
          best = k > best ? k : best;
        }
    }
  }
  if constexpr (TT == TT_LM) {
    best = wave_max_u64(best);
    if (lane == 0) __hip_atomic_fetch_max(&L->lm_best, best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

template <int TT, bool EXACT, bool SHUF>
__device__ __forceinline__ void compute_op(const Params& P, const MegaBufs& M, const Step& S, int k, WBuf (&B)[NB],
                                           int (&t)[NB], const float* page, float* res, int* ids,
                                           const float* resid, const float* rope, MegaLds* L, int lane) {
  const int layer = TT == TT_LM ? P.L : k / 4, count = op_count(P, TT);
  const int n = stream_op<TT, EXACT>(P, layer, count, op_rot<SHUF>(P, k, S.epoch, count), B, t, page, res, ids,
                                     &L->pool[k & 1], lane);
  finish_op<TT>(P, M, S, layer, n, res, ids, resid, rope, L, lane);
}

template <bool EXACT, bool SHUF>
__device__ __forceinline__ void compute_wave(const Params& P, const MegaBufs& M, const Step& S, MegaLds* L,
                                             float* pages, int pf, const float* resid, const float* rope, float* res,
                                             int* ids, int c, int lane, WBuf (&B)[NB], int (&t)[NB], bool more) {
  // on entry the first tasks of operator 0 are in flight (B, t); with `more`
  // (another step follows in this launch) the next step's are put in flight
  // after the LM head
  const int nops = 4 * P.L + 1;
  for (int k = 0; k < nops; ++k) {
    if (!wait_lds(P, M, L, &L->ready[k & 1], (uint32_t)NS * (uint32_t)(k / 2 + 1), NS + c,
                  ((uint32_t)k << 8) | W_READY, lane))
      return;
    const float* page = pages + ((k & 1) ? pf : 0);
    const uint64_t t0 = M.trace ? clock_now() : 0;
    switch (op_type(k, P.L)) {
      case TT_QKV: compute_op<TT_QKV, EXACT, SHUF>(P, M, S, k, B, t, page, res, ids, resid, rope, L, lane); break;
      case TT_O: compute_op<TT_O, EXACT, SHUF>(P, M, S, k, B, t, page, res, ids, resid, rope, L, lane); break;
      case TT_GU: compute_op<TT_GU, EXACT, SHUF>(P, M, S, k, B, t, page, res, ids, resid, rope, L, lane); break;
      case TT_DOWN: compute_op<TT_DOWN, EXACT, SHUF>(P, M, S, k, B, t, page, res, ids, resid, rope, L, lane); break;
      default: compute_op<TT_LM, EXACT, SHUF>(P, M, S, k, B, t, page, res, ids, resid, rope, L, lane); break;
    }
    // the next operator's first tasks go in flight before this one is
    // reported done: the stagers then poll the next input behind the burst
    // of weight loads rather than competing with it.  After QKV the attention
    // path (unit inputs, split records, merged outputs: three hand-overs
    // between workgroups) is the critical path and the O projection's weights
    // are not: their prefetch waits o_delay_ticks after QKV is reported done,
    // so that it does not queue ahead of those hand-overs' reads (it still
    // arrives before the O input does).
    const bool hold = (k & 3) == 0 && k + 1 < nops && P.o_delay_ticks;
    if (hold) {
      if (M.trace && lane == 0) {
        const uint64_t t1 = clock_now();
        M.trace[((size_t)k * gridDim.x + blockIdx.x) * kTraceSlots + c] = ((t1 - t0) << 32) | (uint32_t)t1;
      }
      if (lane == 0) lds_rel_add(&L->done[k & 1], 1u);
      const uint64_t d0 = clock_now();
      while (clock_now() - d0 < P.o_delay_ticks) __builtin_amdgcn_s_sleep(8);
      fetch_first<EXACT, SHUF>(P, k + 1, S.epoch, c, B, t, lane);
      continue;
    }
    if (k + 1 < nops) fetch_first<EXACT, SHUF>(P, k + 1, S.epoch, c, B, t, lane);
    else if (more) fetch_first<EXACT, SHUF>(P, 0, S.epoch + 1, c, B, t, lane);
    if (M.trace && lane == 0) {
      const uint64_t t1 = clock_now();
      M.trace[((size_t)k * gridDim.x + blockIdx.x) * kTraceSlots + c] = ((t1 - t0) << 32) | (uint32_t)t1;
    }
    if (lane == 0) lds_rel_add(&L->done[k & 1], 1u);
  }
  // LM head: the last compute wave of the workgroup publishes the workgroup's key
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(&L->lm_done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
  old = __builtin_amdgcn_readfirstlane(old);
  if (old + 1 == NC && lane == 0) {
    const unsigned long long best = __hip_atomic_load(&L->lm_best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(M.key + blockIdx.x, key_pack(best, S.epoch), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---- stager waves ---------------------------------------------------------------
struct Stager {
  const Params& P;
  const MegaBufs& M;
  const Step& S;
  MegaLds* L;
  int s, lane;     // stager index, lane
  uint32_t gen;    // rendezvous calls so far
  int k;           // operator being staged (for diagnostics)

  __device__ __forceinline__ bool sync() {
    ++gen;
    if (lane == 0) lds_rel_add(&L->ssync, 1u);
    return wait_lds(P, M, L, &L->ssync, (uint32_t)NS * gen, s, ((uint32_t)k << 8) | W_SYNC, lane);
  }
  __device__ __forceinline__ bool wait_done(int op, uint32_t need) {
    return wait_lds(P, M, L, &L->done[op & 1], need, s, ((uint32_t)k << 8) | W_DONE, lane);
  }

  // Words [0, n) of the tagged vector src into dst: this stager takes the
  // 64-word groups s, s + NS, ...; a word is re-read until its tag is current.
  // NORM (RMSNorm input): dst = gain * x, the raw x also into resid when
  // given, and this wave's sum of x^2 into L->red[s] (the compute waves apply
  // the 1/rms factor to the projection outputs).  gain and resid words are
  // the ones this stager owns.
  // While more than a quarter of a batch is stale, a poll round is followed
  // by a longer sleep (two s_sleep 8, about 0.4 us; measured against four and
  // one): most producers are still streaming weights, and the re-reads would
  // only compete with them; once few words are missing the rounds follow each
  // other at once.
  template <bool NORM = false>
  __device__ __forceinline__ bool load_tagged(const uint64_t* src, int n, float* dst, const float* gain = nullptr,
                                              float* resid = nullptr) {
    constexpr int BATCH = 28;
    const uint32_t ep = S.epoch;
    float ss = 0.f;
    mark(k, NC + 1);
    for (int g0 = s; g0 * kWave < n; g0 += NS * BATCH) {
      uint64_t w[BATCH];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int i = (g0 + j * NS) * kWave + lane;
        w[j] = i < n ? tget(src + i) : ((uint64_t)ep << 32);
      }
      Spin sp;
      for (;;) {
        uint32_t pend = 0;
#pragma unroll
        for (int j = 0; j < BATCH; ++j) pend |= tcur(w[j], ep) ? 0u : 1u << j;
        if (__builtin_amdgcn_ballot_w64(pend != 0) == 0) break;
        const float stale = wave_sum((float)__popc(pend));  // exact: at most BATCH * 64
        if (!sp.tick<kPollSleep>(P, M, L, s, ((uint32_t)k << 8) | W_DATA, (uint32_t)g0, (uint32_t)n, lane)) return false;
        if (stale * 4.0f > (float)(BATCH * kWave)) {
#pragma unroll
          for (int z = 0; z < 2; ++z) __builtin_amdgcn_s_sleep(8);
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j)
          if ((pend >> j) & 1) w[j] = tget(src + (g0 + j * NS) * kWave + lane);
      }
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int i = (g0 + j * NS) * kWave + lane;
        if (i < n) {
          const float v = tval(w[j]);
          if constexpr (NORM) {
            if (resid) resid[i] = v;
            dst[i] = v * gain[i];
            ss = fmaf(v, v, ss);
          } else {
            dst[i] = v;
          }
        }
      }
    }
    if constexpr (NORM) {
      ss = wave_sum(ss);
      if (lane == 0) L->red[s] = ss;
    }
    mark(k, NC + 2);
    return true;
  }

  // The bf16 embedding row of the step's token (read-only data, plain loads)
  // as an RMSNorm input: page = gain * x, raw x into resid, sum of x^2 into
  // L->red[s].
  // The step's token: from the caller's array, or (a later step of a
  // multi-step launch, S.tokens null) the previous step's greedy id, a tagged
  // word written by workgroup 0's argmax.
  __device__ __forceinline__ bool step_token(int* tok) {
    if (S.tokens) {
      *tok = token_of(P, S, 0);
      return true;
    }
    const uint64_t need = (uint64_t)(S.epoch - 1) << 32;
    uint64_t w = tget(M.tok);
    Spin sp;
    while ((w >> 32) != (need >> 32)) {
      if (!sp.tick<kPollSleep>(P, M, L, s, ((uint32_t)k << 8) | W_KEY, 0u, 1u, lane)) return false;
      w = tget(M.tok);
    }
    const int t = (int)(uint32_t)w;
    *tok = t >= 0 && t < P.V ? t : 0;
    return true;
  }

  __device__ __forceinline__ void load_embed(float* dst, const float* gain, float* resid, int tok) {
    const uint16_t* row = P.embed + (int64_t)tok * P.H;
    float ss = 0.f;
    for (int i = (s * kWave + lane); i < P.H; i += NS * kWave) {
      const float v = bf1(row[i]);
      resid[i] = v;
      dst[i] = v * gain[i];
      ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) L->red[s] = ss;
  }

  // This stager's RMSNorm gains (words s*64 + lane + 256 j) into the LDS gain
  // buffer, loaded while nothing waits on them: staging a normalised input
  // then needs no global load after the input has arrived.  Each stager reads
  // back only the words it wrote.
  __device__ __forceinline__ void load_gain(const uint16_t* gamma, int n, float* gain) {
    for (int i = s * kWave + lane; i < n; i += NS * kWave) gain[i] = bf1(gamma[i]);
  }

  __device__ __forceinline__ void mark(int op, int slot) {
    if (M.trace && s == 0 && lane == 0)
      M.trace[((size_t)op * gridDim.x + blockIdx.x) * kTraceSlots + slot] = clock_now();
  }

  // This stager's part of op's input (and its L->red word) is in the page:
  // ready[page] counts the stagers' releases, NS per operator on the page.
  __device__ __forceinline__ void publish(int op, int page) {
    if (lane == 0) {
      if (s == 0) {
        L->pool[page] = NB * NC;  // pool slots past the compute waves' first NB tasks
        if (M.trace) M.trace[((size_t)op * gridDim.x + blockIdx.x) * kTraceSlots + NC] = clock_now();
      }
      lds_rel_add(&L->ready[page], 1u);
    }
  }
};

// Log-sum-exp merge of query head hq's split records -> tagged attention
// output, by the workgroup's NS stager waves together.  Wave s takes the
// splits s, s + NS, s + 2 NS, ..., SB of them per round: every load of a
// round (this lane's dims of each split's o, and its (m, l) for lane < SB) is
// issued at once, then only stale words are read again, so up to NS SB
// splits cost one round trip.  Each wave merges its splits online (running
// maximum, rescaled sums); the NS partial states then meet in LDS, where
// wave 0 combines them in wave order and writes the output.
template <int HD>
__device__ __forceinline__ bool merge_unit(Stager& st, int l, int hq, float* recs) {
  const Params& P = st.P;
  const MegaBufs& M = st.M;
  const int lane = st.lane, s = st.s, G = P.nq / P.nkv, g = hq / G, hh = hq % G;
  const int used = (st.S.pos + 1 + P.split - 1) / P.split;
  constexpr int DPL = HD / kWave, SB = 8;
  const uint32_t ep = st.S.epoch;
  const uint64_t cur = (uint64_t)ep << 32;
  const size_t rs = (size_t)G * (HD + 2);
  const uint64_t* base = M.rec + ((size_t)l * P.nkv + g) * P.nsplit * rs + (size_t)hh * (HD + 2);
  float Mx = -INFINITY, Lsum = 0.f, o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  for (int s0 = 0; s0 < used; s0 += NS * SB) {
    // this wave's splits of the round: s0 + s + NS j, j < n
    const int first = s0 + s, n = first < used ? min(SB, (used - first + NS - 1) / NS) : 0;
    const bool mine = lane < n;  // this lane reads split first + NS lane's (m, l)
    const uint64_t* ml = base + (size_t)(first + NS * (mine ? lane : 0)) * rs + HD;
    uint64_t wm = mine ? tget(ml) : cur, wl = mine ? tget(ml + 1) : cur, w[SB][DPL];
#pragma unroll
    for (int j = 0; j < SB; ++j)
#pragma unroll
      for (int e = 0; e < DPL; ++e)
        w[j][e] = j < n ? tget(base + (size_t)(first + NS * j) * rs + lane * DPL + e) : cur;
    Spin sp;
    for (;;) {
      bool ok = tcur(wm, ep) && tcur(wl, ep);
#pragma unroll
      for (int j = 0; j < SB; ++j)
#pragma unroll
        for (int e = 0; e < DPL; ++e) ok = ok && tcur(w[j][e], ep);
      if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
      if (!sp.tick<kPollSleep>(P, M, st.L, s, ((uint32_t)st.k << 8) | W_REC, (uint32_t)s0, (uint32_t)used, lane))
        return false;
      if (!tcur(wm, ep)) wm = tget(ml);
      if (!tcur(wl, ep)) wl = tget(ml + 1);
#pragma unroll
      for (int j = 0; j < SB; ++j)
#pragma unroll
        for (int e = 0; e < DPL; ++e)
          if (!tcur(w[j][e], ep)) w[j][e] = tget(base + (size_t)(first + NS * j) * rs + lane * DPL + e);
    }
    // records with l == 0 hold no positions and carry weight 0
    const float ms = tval(wm), ls = tval(wl);
    const bool live = mine && ls > 0.f;
    const float Mn = fmaxf(Mx, wave_max(live ? ms : -INFINITY));
    if (Mn == -INFINITY) continue;  // nothing live yet
    const float alpha = Mx == -INFINITY ? 0.f : __expf(Mx - Mn);
    const float wgt = live ? __expf(ms - Mn) : 0.f;
    Lsum = Lsum * alpha + wave_sum(wgt * (live ? ls : 0.f));
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const float wj = __shfl(wgt, j);
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = fmaf(wj, wj > 0.f ? tval(w[j][e]) : 0.f, o[e]);
    }
    Mx = Mn;
  }
  st.mark(st.k, NC + 5);
  float* mine_rec = recs + s * (HD + 2);
#pragma unroll
  for (int e = 0; e < DPL; ++e) mine_rec[lane * DPL + e] = o[e];
  if (lane == 0) {
    mine_rec[HD] = Mx;
    mine_rec[HD + 1] = Lsum;
  }
  if (!st.sync()) return false;  // every wave's state is in recs
  if (s == 0) {
    float Mt = -INFINITY, Lt = 0.f, ot[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) ot[e] = 0.f;
#pragma unroll
    for (int w = 0; w < NS; ++w) {
      const float* r = recs + w * (HD + 2);
      const float lw = r[HD + 1];
      if (!(lw > 0.f)) continue;
      const float mw = r[HD], Mn = fmaxf(Mt, mw);
      const float a = __expf(Mt - Mn), c = __expf(mw - Mn);
      Lt = Lt * a + lw * c;
#pragma unroll
      for (int e = 0; e < DPL; ++e) ot[e] = ot[e] * a + r[lane * DPL + e] * c;
      Mt = Mn;
    }
    const float inv = 1.0f / Lt;
    uint64_t* out = M.attn + (size_t)l * P.nq * HD + (size_t)hq * HD + lane * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) tput(out + e, ot[e] * inv, ep);
    st.mark(st.k, NC + 6);
  }
  return st.sync();  // recs is reused by the next merge
}

// Puts the key of row jr of a block held in registers (the current position,
// whose key arrives as tagged words this step) into the block: kv holds this
// lane's dims lane * DPL + e.  The key part a lane scores (dims part * EPL ..)
// is gathered from the lanes that hold those dims; every lane takes part in
// the shuffles, the lanes of row jr keep them.  (The row's value is taken
// from registers when the block is computed.)
template <int HD, typename KT>
__device__ __forceinline__ void attn_patch_k(AttnBuf<HD, KT>& A, int jr, const float (&kv)[HD / kWave], int lane) {
  using Gm = AttnGeom<HD, KT>;
  constexpr int DPL = Gm::DPL, EPL = Gm::EPL;
  const int my = lane / Gm::LPP, part = lane % Gm::LPP;
  float kp[EPL];
#pragma unroll
  for (int m = 0; m < EPL; ++m) kp[m] = __shfl(kv[m % DPL], (part * EPL + m) / DPL);
  if (my == jr) {
#pragma unroll
    for (int i = 0; i < Gm::KV16; ++i) {
      if constexpr (sizeof(KT) == 4) {
        A.kr[i] = v4u{__float_as_uint(kp[4 * i]), __float_as_uint(kp[4 * i + 1]), __float_as_uint(kp[4 * i + 2]),
                      __float_as_uint(kp[4 * i + 3])};
      } else {
        A.kr[i] = v4u{bf_pack(f2bf(kp[8 * i]), f2bf(kp[8 * i + 1])), bf_pack(f2bf(kp[8 * i + 2]), f2bf(kp[8 * i + 3])),
                      bf_pack(f2bf(kp[8 * i + 4]), f2bf(kp[8 * i + 5])), bf_pack(f2bf(kp[8 * i + 6]), f2bf(kp[8 * i + 7]))};
      }
    }
  }
}

// One decode-attention unit: the G query heads of KV head g over the split
// [p0, p1) of the context, as one (o, m, l) record per head.  The workgroup's
// NS stager waves share the unit: wave s takes the position blocks s, s + NS,
// ... (one block each at the split sizes used), keeps an online-softmax state
// per head, and the waves' states are merged through LDS.  A wave's first
// block is loaded from the cache before the queries are awaited: rows below
// the current position depend on nothing this step writes, and the current
// position's row (the block clamps at it) is put into the registers from its
// tagged key and value once they arrive; that wave also appends the row to
// the cache for later steps.  A (KV head, split) unit always runs on the same
// workgroup, so every cache row this launch writes is read back only by the
// workgroup that wrote it.
template <int HD, typename KT, int GQ>
__device__ __forceinline__ bool attn_unit(Stager& st, int l, int g, int sp_i, float* qs, float* recs) {
  const Params& P = st.P;
  const MegaBufs& M = st.M;
  const int lane = st.lane, s = st.s, T = st.S.pos + 1;
  constexpr int G = GQ, DPL = HD / kWave, NP = AttnGeom<HD, KT>::NP;
  const int p0 = sp_i * P.split, p1 = min(p0 + P.split, T);
  const uint32_t ep = st.S.epoch;
  const int qd = P.nq * HD, kd = P.nkv * HD;
  const uint64_t* qkv = M.qkv + (size_t)l * (qd + 2 * kd);
  const uint64_t cur = (uint64_t)ep << 32;
  // The group's queries (G * HD words, shared by the waves: this wave loads
  // every NS-th 64-word group) and, for the block that holds the current
  // position, its key and value; all loads issued at once, then only stale
  // words are read again.
  constexpr int QW = (G * HD / kWave + NS - 1) / NS;
  const uint64_t* qsrc = qkv + (size_t)g * G * HD + lane;
  const int last_blk = (T - 1 - p0) / NP;  // block (within the split) of position T - 1, if p1 == T
  const bool append = p1 == T && last_blk % NS == s;
  const uint64_t* ks = qkv + qd + (size_t)g * HD + lane * DPL;
  const uint64_t* vs = qkv + qd + kd + (size_t)g * HD + lane * DPL;
  const int64_t o0 = kv_off(P, l, 0, g, 0);
  KT* kc = static_cast<KT*>(P.kcache) + o0;
  KT* vc = static_cast<KT*>(P.vcache) + o0;
  // this wave's first block: its keys from the cache (clamped at the current
  // position) before the queries are awaited, its values once they are here
  // (values are used after the scores, so their loads overlap the softmax)
  int b0 = p0 + s * NP;
  AttnBuf<HD, KT> A;
  bool pre = b0 < p1;
  if (pre) attn_load_k<HD, KT>(kc, b0, p1, lane, A);
  uint64_t qw[QW], kw[DPL], vw[DPL];
#pragma unroll
  for (int j = 0; j < QW; ++j) qw[j] = (s + j * NS) * kWave < G * HD ? tget(qsrc + (s + j * NS) * kWave) : cur;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    kw[e] = append ? tget(ks + e) : cur;
    vw[e] = append ? tget(vs + e) : cur;
  }
  {
    Spin sp;
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int j = 0; j < QW; ++j) ok = ok && tcur(qw[j], ep);
#pragma unroll
      for (int e = 0; e < DPL; ++e) ok = ok && tcur(kw[e], ep) && tcur(vw[e], ep);
      if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
      if (!sp.tick<kPollSleep>(P, M, st.L, s, ((uint32_t)st.k << 8) | W_QKV, (uint32_t)(g * P.nsplit + sp_i), 0u, lane))
        return false;
#pragma unroll
      for (int j = 0; j < QW; ++j)
        if (!tcur(qw[j], ep)) qw[j] = tget(qsrc + (s + j * NS) * kWave);
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        if (!tcur(kw[e], ep)) kw[e] = tget(ks + e);
        if (!tcur(vw[e], ep)) vw[e] = tget(vs + e);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < QW; ++j)
    if ((s + j * NS) * kWave < G * HD) qs[(s + j * NS) * kWave + lane] = tval(qw[j]);
  float vf[DPL];  // the current position's value (this lane's dims), when this wave appends
  int jr = -1;    // its row in the first block, if there
  if (append) {  // position T - 1: into the cache for later steps, into the first block for this one
    float kf[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      kf[e] = tval(kw[e]);
      vf[e] = tval(vw[e]);
      const int64_t at = (int64_t)(T - 1) * HD + lane * DPL + e;
      if constexpr (sizeof(KT) == 4) { kc[at] = kf[e]; vc[at] = vf[e]; }
      else { kc[at] = f2bf(kf[e]); vc[at] = f2bf(vf[e]); }
    }
    if (T - 1 - b0 < NP) {
      jr = T - 1 - b0;
      attn_patch_k<HD, KT>(A, jr, kf, lane);  // the row is in the first block
    } else {
      // the row is in a later block of this wave, loaded below by other lanes
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  }
  if (pre) attn_load_v<HD, KT>(vc, b0, p1, lane, A);
  st.mark(st.k, NC + 3);
  if (!st.sync()) return false;  // every wave's query words are in qs
  st.mark(st.k, NC + 7);
  AttnState<HD, GQ> sta;
  sta.init();
  if (pre) {
    attn_compute<HD, KT, GQ>(A, qs, b0, p1, G, lane, sta, jr, vf);
    b0 += NS * NP;
  }
  for (; b0 < p1; b0 += NS * NP) {
    attn_load<HD, KT>(kc, vc, b0, p1, lane, A);
    attn_compute<HD, KT, GQ>(A, qs, b0, p1, G, lane, sta);
  }
  attn_store_state<HD, GQ>(sta, G, recs + s * G * (HD + 2), lane);
  st.mark(st.k, NC + 8);
  if (!st.sync()) return false;  // every wave's state is in recs
  st.mark(st.k, NC + 9);
  // merge the waves' states of head h (wave h % NS) into the unit's record
  uint64_t* rec = M.rec + (((size_t)l * P.nkv + g) * P.nsplit + sp_i) * G * (HD + 2);
  for (int h = s; h < G; h += NS) {
    float Mx = -INFINITY, Ls = 0.f, o[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = 0.f;
#pragma unroll
    for (int w = 0; w < NS; ++w) {
      const float* r = recs + (w * G + h) * (HD + 2);
      const float lw = r[HD + 1];
      if (!(lw > 0.f)) continue;
      const float mw = r[HD], Mn = fmaxf(Mx, mw);
      const float a = __expf(Mx - Mn), c = __expf(mw - Mn);
      Ls = Ls * a + lw * c;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = o[e] * a + r[lane * DPL + e] * c;
      Mx = Mn;
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) tput(rec + h * (HD + 2) + lane * DPL + e, o[e], ep);
    if (lane == 0) {
      tput(rec + h * (HD + 2) + HD, Mx, ep);
      tput(rec + h * (HD + 2) + HD + 1, Ls, ep);
    }
  }
  st.mark(st.k, NC + 4);
  return st.sync();  // qs and recs are reused by the next unit
}

// The step's greedy token from every workgroup's LM-head key.
__device__ __forceinline__ bool argmax_unit(Stager& st) {
  const Params& P = st.P;
  const MegaBufs& M = st.M;
  const int lane = st.lane, n = gridDim.x;
  const uint32_t tag = st.S.epoch & 0x7FFFu;
  uint64_t best = 0;
  for (int i0 = 0; i0 < n; i0 += kWave) {
    const int i = min(i0 + lane, n - 1);
    uint64_t w = tget(M.key + i);
    Spin sp;
    while (__builtin_amdgcn_ballot_w64((w & 0x7FFFu) != tag) != 0) {
      if (!sp.tick<kPollSleep>(P, M, st.L, st.s, ((uint32_t)st.k << 8) | W_KEY, (uint32_t)i0, (uint32_t)n, lane)) return false;
      if ((w & 0x7FFFu) != tag) w = tget(M.key + i);
    }
    best = (w >> 15) > best ? (w >> 15) : best;
  }
  best = wave_max_u64(best);
  if (lane == 0) {
    const uint32_t idx = 0x1FFFFu - (uint32_t)(best & 0x1FFFFu);
    const unsigned long long k = ((best >> 17) << 32) | (0xFFFFFFFFu - idx);
    st.S.out[0] = (int32_t)idx;
    // the next step of the same launch starts from this id
    __hip_atomic_store(M.tok, ((uint64_t)st.S.epoch << 32) | idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!(fabsf(argmax_key_value(k)) <= 3.0e38f)) atomicCAS(&P.status[1], ST_OK, ST_NONFINITE);
  }
  return true;
}

template <int HD, typename KT, int GQ>
__device__ __forceinline__ void stager_wave(const Params& P, const MegaBufs& M, const Step& S, MegaLds* L,
                                            float* pages, int pf, float* resid, float* gain, float* rope, float* qs,
                                            float* recs, int s, int lane) {
  Stager st{P, M, S, L, s, lane, 0u, 0};
  const int Lc = P.L, ncu = gridDim.x, wg = blockIdx.x;
  const int nunits = P.nkv * P.nsplit, used = (S.pos + 1 + P.split - 1) / P.split;
  static_assert(GQ >= 1 && GQ <= kMaxGqa, "query heads per KV head");
  // RoPE angles of this position (host-computed table, read-only)
  const int half = P.hd / 2;
  for (int i = s * kWave + lane; i < half; i += NS * kWave) {
    rope[i] = P.rope_cos[(int64_t)S.pos * half + i];
    rope[half + i] = P.rope_sin[(int64_t)S.pos * half + i];
  }
  float* page0 = pages;
  float* page1 = pages + pf;  // page 0 holds hidden-size inputs only
  for (int l = 0; l < Lc; ++l) {
    int k = 4 * l;
    // QKV: rmsnorm(x_l) (layer 0: the embedding row), raw x_l kept for the O residual
    st.k = k;
    if (l == 0) st.load_gain(ld_const(P.attn_norm), P.H, gain);  // later layers: loaded during the previous DOWN
    if (!st.wait_done(k, free_for(k))) return;
    if (l == 0) {
      int tok = 0;
      if (!st.step_token(&tok)) return;
      st.load_embed(page0, gain, resid, tok);
    }
    else if (!st.wait_done(k - 1, done_after(k - 1)) ||
             !st.load_tagged<true>(M.x + (size_t)l * P.H, P.H, page0, gain, resid))
      return;
    st.publish(k, 0);
    // attention units of this workgroup (all stager waves), then the
    // log-sum-exp merges of the query heads assigned to this wave; both wait
    // for the local QKV tasks first, so that they do not poll while QKV runs
    st.load_gain(ld_const(P.ffn_norm + l), P.H, gain);  // for GU, ahead of every wait below
    const int hq0 = ncu - 1 - wg;  // query heads merged here: hq0, hq0 + ncu, ... (all stager waves)
    st.k = k + 1;  // attention and merges are traced under the O operator
    if (wg < nunits || hq0 < P.nq)
      if (!st.wait_done(k, done_after(k))) return;
    for (int u = wg; u < nunits; u += ncu) {
      const int g = u / P.nsplit, sp_i = u % P.nsplit;
      if (sp_i >= used) continue;
      if (!attn_unit<HD, KT, GQ>(st, l, g, sp_i, qs, recs)) return;
    }
    for (int hq = hq0; hq < P.nq; hq += ncu)
      if (!merge_unit<HD>(st, l, hq, recs)) return;
    // O: the merged attention output
    st.k = ++k;
    if (!st.wait_done(k, free_for(k)) || !st.load_tagged(M.attn + (size_t)l * P.nq * P.hd, P.nq * P.hd, page1))
      return;
    st.publish(k, 1);
    // GU: rmsnorm(xmid), raw xmid kept for the down residual
    st.k = ++k;
    if (!st.wait_done(k, free_for(k)) || !st.wait_done(k - 1, done_after(k - 1)) ||
        !st.load_tagged<true>(M.xmid + (size_t)l * P.H, P.H, page0, gain, resid))
      return;
    st.publish(k, 0);
    // DOWN: the SwiGLU output
    st.k = ++k;
    if (l + 1 < Lc) st.load_gain(ld_const(P.attn_norm + l + 1), P.H, gain);  // for the next QKV
    else st.load_gain(P.final_norm, P.H, gain);                               // for the LM head
    if (!st.wait_done(k, free_for(k)) || !st.wait_done(k - 1, done_after(k - 1)) ||
        !st.load_tagged(M.h + (size_t)l * P.F, P.F, page1))
      return;
    st.publish(k, 1);
  }
  // LM head: rmsnorm(x_L)
  const int k = 4 * Lc;
  st.k = k;
  if (!st.wait_done(k, free_for(k)) || !st.wait_done(k - 1, done_after(k - 1)) ||
      !st.load_tagged<true>(M.x + (size_t)Lc * P.H, P.H, page0, gain, nullptr))
    return;
  st.publish(k, 0);
  if (wg == 0 && s == 1) {
    st.k = k + 1;
    if (!st.wait_done(k, done_after(k))) return;
    argmax_unit(st);
  }
}

template <bool EXACT, int HD, typename KT, int GQ, bool SHUF>
__device__ __forceinline__ void mega_body(const Params& P, const MegaBufs& M, const Step& S, int) {
  extern __shared__ __align__(16) unsigned char smem[];
  MegaLds* L = reinterpret_cast<MegaLds*>(smem);
  float* pages = reinterpret_cast<float*>(smem + sizeof(MegaLds));
  int pf, pf1;
  mega_pages(P.H, P.nq * HD, P.F, &pf, &pf1);
  float* resid = pages + pf + pf1;
  float* gain = resid + ((P.H + 3) & ~3);
  float* rope = gain + ((P.H + 3) & ~3);
  float* res = rope + ((HD + 3) & ~3);
  constexpr int rs = kMegaMaxTasks * (kR + 1);  // per compute wave: results + task ids
  float* qs = res + NC * rs;                     // attention unit: the group's queries [GQ][HD]
  float* recs = qs + GQ * HD;                    // attention unit: the waves' states [NS][GQ][HD + 2]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nst = S.nsteps > 0 ? S.nsteps : 1;
  // Step i of the launch; the LDS counters start again from zero at every
  // step (wave 0 resets them after the barrier that ends the previous step).
  auto begin_step = [&](int i, Step& Si) __attribute__((always_inline)) -> bool {
    if (threadIdx.x == 0) {
      L->ready[0] = L->ready[1] = 0;
      L->done[0] = L->done[1] = 0;
      L->pool[0] = L->pool[1] = 0;
      L->ssync = 0;
      L->lm_done = 0;
      L->lm_best = 0;
      if (i == 0) L->abort = __hip_atomic_load(&P.status[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ? 1u : 0u;
    }
    __syncthreads();
    if (L->abort) return false;  // the same decision in every wave of the workgroup
    Si = S;
    Si.epoch = S.epoch + (uint32_t)i;
    Si.pos = S.pos + i;
    Si.tokens = S.tok_step ? S.tokens + (int64_t)i * S.tok_step : (i == 0 ? S.tokens : nullptr);
    Si.out = S.out + (int64_t)i * S.out_step;
    Si.logits = i + 1 == nst ? S.logits : nullptr;
    return true;
  };
  // The two roles run the same sequence of workgroup barriers (two per step)
  // in separate loops, so that neither role's registers are live in the
  // other's code.  A wave that stopped early (abort) still reaches the
  // step's closing barrier: every wait sees the abort word, so the whole
  // workgroup arrives.
  if (wave < NS) {
    for (int i = 0; i < nst; ++i) {
      Step Si;
      if (!begin_step(i, Si)) return;
      stager_wave<HD, KT, GQ>(P, M, Si, L, pages, pf, resid, gain, rope, qs, recs, wave, lane);
      __syncthreads();
    }
  } else {
    const int c = wave - NS;
    float* r = res + c * rs;
    WBuf B[NB];  // the next operator's first tasks, in flight across operators and steps
    int t[NB];
    fetch_first<EXACT, SHUF>(P, 0, S.epoch, c, B, t, lane);
    for (int i = 0; i < nst; ++i) {
      Step Si;
      if (!begin_step(i, Si)) return;
      compute_wave<EXACT, SHUF>(P, M, Si, L, pages, pf, resid, rope, r, reinterpret_cast<int*>(r + kMegaMaxTasks * kR), c,
                          lane, B, t, i + 1 < nst);
      __syncthreads();
    }
  }
}

}  // namespace

// S.nsteps decode steps of one sequence, per (EXACT, head_dim, cache element
// type, query heads per KV head).  EXACT: every GEMV operator's K is a multiple of
// 512 with a chunk count that is a multiple of the in-flight depth (no
// clamped loads).  The generic (n) instances also deal tasks in the order
// MK_FLAG_SHUFFLE asks for; the exact (x) ones, which the production shapes
// run, carry no rotation at all.  The host picks the instance (mega_kernel).
#define MK_MEGA(X, HD, KN, KT, G)                                                                          \
  extern "C" __global__ __launch_bounds__(kMegaWaves * kWave) void mk_mega_##X##_##HD##_##KN##_g##G(       \
      Params P, MegaBufs M, Step S, int pf) {                                                              \
    mega_body<X##_EXACT, HD, KT, G, X##_SHUF>(P, M, S, pf);                                                \
  }
#define x_EXACT true
#define n_EXACT false
#define x_SHUF false
#define n_SHUF true
#define MK_MEGA_G(X, HD, KN, KT) MK_MEGA(X, HD, KN, KT, 1) MK_MEGA(X, HD, KN, KT, 2) MK_MEGA(X, HD, KN, KT, 4) \
  MK_MEGA(X, HD, KN, KT, 8)
#if MK_MEGA_PART == 0
MK_MEGA_G(n, 64, f32, float)
MK_MEGA_G(n, 64, bf16, uint16_t)
#elif MK_MEGA_PART == 1
MK_MEGA_G(n, 128, f32, float)
MK_MEGA_G(n, 128, bf16, uint16_t)
#else
MK_MEGA(x, 64, f32, float, 4)
MK_MEGA(x, 64, bf16, uint16_t, 4)
MK_MEGA(x, 128, f32, float, 4)
MK_MEGA(x, 128, bf16, uint16_t, 4)
// the LDS layout, once
int mega_lds_bytes(int H, int nq, int nkv, int hd, int F, int* page_floats) {
  int pf0, pf1;
  mega_pages(H, nq * hd, F, &pf0, &pf1);
  if (page_floats) *page_floats = pf0 + pf1;
  const int G = nq / nkv;
  const int floats = pf0 + pf1 + 2 * ((H + 3) & ~3) + ((hd + 3) & ~3) + NC * kMegaMaxTasks * (kR + 1) + G * hd +
                     NS * G * (hd + 2);
  return (int)sizeof(MegaLds) + 4 * floats;
}
#endif
#undef MK_MEGA_G
#undef n_EXACT
#undef x_EXACT
#undef n_SHUF
#undef x_SHUF
#undef MK_MEGA

}  // namespace mk
