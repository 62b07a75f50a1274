// Device entry points: the persistent megakernel (scheduler wave + worker
// waves per CU), the kernel-per-operator baseline built from the same task
// bodies, and single-body kernels used by the unit tests.
//
// Runtime design (after "Compilar LLM en un MegaKernel ...", section "Parte 2.
// Runtime", and "MPK: A Compiler and Runtime ...", sections 3-4), re-cut for
// CDNA4: one workgroup per CU; wave 0 is the CU's scheduler, waves 1..7 are
// workers.  The host places every task on a per-CU queue ahead of time.  A
// worker takes the next queue ticket as soon as it is free and starts
// streaming that task's weights (they depend on no event), then waits until
// the scheduler's ready frontier passes its ticket.  The scheduler walks the
// queue in order: it waits for each task's input event in global memory
// (counter >= threshold * epoch, agent-scope acquire), stages the task's input
// activation vector into one of two LDS pages (computing the RMSNorm on the
// way), and advances the frontier.  A finished task bumps a per-CU LDS counter;
// the last task of a run of same-event tasks releases at agent scope and adds
// one to the global event counter.
#include "device.h"
#include "kernels.h"

namespace mk {

__device__ __forceinline__ int64_t kv_off(const Params& P, int l, int b, int g, int p) {
  return ((((int64_t)l * P.B + b) * P.nkv + g) * P.max_seq + p) * P.hd;
}

// Token id of batch row b, clamped into [0, V) so that a bad id can never
// address outside the embedding table; a clamp latches ST_BADTOKEN.
__device__ __forceinline__ int token_of(const Params& P, const Step& S, int b) {
  const int t = S.tokens[(int64_t)b * S.tok_stride];
  if (t >= 0 && t < P.V) return t;
  atomicCAS(&P.status[1], ST_OK, ST_BADTOKEN);
  return 0;
}

// Source of a staged input vector.
__device__ void stage_input(const Params& P, const Step& S, uint16_t key, int b, float* page, int lane) {
  const int kind = stage_kind(key), l = stage_layer(key);
  const int64_t H = P.H;
  switch (kind) {
    case SK_ATTN_NORM:
      if (l == 0) stage_vector(page, nullptr, P.embed + (int64_t)token_of(P, S, b) * H, P.H, P.attn_norm[0], P.eps, lane);
      else stage_vector(page, P.xs + ((int64_t)l * P.B + b) * H, nullptr, P.H, P.attn_norm[l], P.eps, lane);
      break;
    case SK_O_IN: {
      const int n = P.nq * P.hd;
      stage_vector(page, P.attn_out + ((int64_t)l * P.B + b) * n, nullptr, n, nullptr, 0.f, lane);
      break;
    }
    case SK_FFN_NORM:
      stage_vector(page, P.xmid + ((int64_t)l * P.B + b) * H, nullptr, P.H, P.ffn_norm[l], P.eps, lane);
      break;
    case SK_H:
      stage_vector(page, P.h + ((int64_t)l * P.B + b) * P.F, nullptr, P.F, nullptr, 0.f, lane);
      break;
    default:
      stage_vector(page, P.xs + ((int64_t)P.L * P.B + b) * H, nullptr, P.H, P.final_norm, P.eps, lane);
      break;
  }
}

__device__ __forceinline__ float pick4(const float (&y)[kRows], int i) {
  return i == 0 ? y[0] : i == 1 ? y[1] : i == 2 ? y[2] : y[3];
}

// Runs one task on one wave.  `wait()` is called after the weight prefetch and
// before anything that reads activations; it returns false on abort.
template <class Wait>
__device__ bool exec_task(const Params& P, const Step& S, const Task& d, int lane, const float* page, float* scratch,
                          Lds* L, Wait wait) {
  const int l = d.layer, b = d.batch;
  switch (d.type) {
    case TT_QKV: case TT_O: case TT_GU: case TT_DOWN: case TT_LM: {
      GemvRows g;
      const uint16_t* W;
      int K = P.H;
      g.mask = 0;
      if (d.type == TT_QKV) {
        W = d.a0 == 0 ? P.wq[l] : d.a0 == 1 ? P.wk[l] : P.wv[l];
        if (d.a3) {
          const int np = d.a2 / 2;
          for (int j = 0; j < 2; ++j) {
            g.row[j] = reinterpret_cast<const v4u*>(W + (int64_t)(d.a1 + j) * K);
            g.row[2 + j] = reinterpret_cast<const v4u*>(W + (int64_t)(d.a1 + d.a3 + j) * K);
            if (j < np) g.mask |= (1u << j) | (1u << (2 + j));
          }
        } else {
          for (int j = 0; j < kRows; ++j) {
            g.row[j] = reinterpret_cast<const v4u*>(W + (int64_t)(d.a1 + j) * K);
            if (j < d.a2) g.mask |= 1u << j;
          }
        }
      } else if (d.type == TT_GU) {
        for (int j = 0; j < 2; ++j) {
          g.row[j] = reinterpret_cast<const v4u*>(P.w_gate[l] + (int64_t)(d.a1 + j) * K);
          g.row[2 + j] = reinterpret_cast<const v4u*>(P.w_up[l] + (int64_t)(d.a1 + j) * K);
          if (j < d.a2) g.mask |= (1u << j) | (1u << (2 + j));
        }
      } else {
        if (d.type == TT_O) { W = P.wo[l]; K = P.nq * P.hd; }
        else if (d.type == TT_DOWN) { W = P.w_down[l]; K = P.F; }
        else W = P.tied ? P.embed : P.lm_head;
        for (int j = 0; j < kRows; ++j) {
          g.row[j] = reinterpret_cast<const v4u*>(W + (int64_t)(d.a1 + j) * K);
          if (j < d.a2) g.mask |= 1u << j;
        }
      }
      g.nvec = K / 8;
      v4u buf[kDepth][kRows];
      gemv_prefetch(buf, g, lane);
      if (!wait()) return false;
      float y[kRows];
      gemv_run(buf, g, page, lane, y);
      // epilogues: lane r handles row slot r
      const int r = lane;
      if (r < kRows && ((g.mask >> r) & 1)) {
        const float v = pick4(y, r);
        const int64_t H = P.H;
        switch (d.type) {
          case TT_QKV: {
            if (d.a3) {
              const int half = P.hd / 2, j = r & 1;
              const float lo = pick4(y, j), hi = pick4(y, 2 + j);
              const int i = (d.a1 % P.hd) + j;
              const float c = P.rope_cos[(int64_t)S.pos * half + i], s = P.rope_sin[(int64_t)S.pos * half + i];
              const float rot = r < 2 ? lo * c - hi * s : hi * c + lo * s;
              const int row = r < 2 ? d.a1 + j : d.a1 + d.a3 + j;
              if (d.a0 == 0) {
                P.q[((int64_t)l * P.B + b) * P.nq * P.hd + row] = rot;
              } else {
                const int grp = row / P.hd;
                P.kcache[kv_off(P, l, b, grp, S.pos) + row % P.hd] = f2bf(rot);
              }
            } else {
              const int row = d.a1 + r, grp = row / P.hd;
              P.vcache[kv_off(P, l, b, grp, S.pos) + row % P.hd] = f2bf(v);
            }
            break;
          }
          case TT_O: {
            const int row = d.a1 + r;
            const float xin = l == 0 ? bf1(P.embed[(int64_t)token_of(P, S, b) * H + row])
                                     : P.xs[((int64_t)l * P.B + b) * H + row];
            P.xmid[((int64_t)l * P.B + b) * H + row] = xin + v;
            break;
          }
          case TT_GU:
            if (r < 2) P.h[((int64_t)l * P.B + b) * P.F + d.a1 + r] = silu(v) * pick4(y, r + 2);
            break;
          case TT_DOWN: {
            const int row = d.a1 + r;
            P.xs[((int64_t)(l + 1) * P.B + b) * H + row] = P.xmid[((int64_t)l * P.B + b) * H + row] + v;
            break;
          }
          default: {  // TT_LM
            const int row = d.a1 + r;
            if (S.logits) S.logits[(int64_t)b * P.V + row] = v;
            break;
          }
        }
      }
      if (d.type == TT_LM) {
        unsigned long long best = 0;
        for (int j = 0; j < kRows; ++j)
          if ((g.mask >> j) & 1) {
            const unsigned long long k = argmax_key(pick4(y, j), (uint32_t)(d.a1 + j));
            best = k > best ? k : best;
          }
        if (lane == 0) __hip_atomic_fetch_max(&L->lm_best[b], best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      break;
    }
    case TT_ATTN: {
      if (!wait()) return false;
      const int G = P.nq / P.nkv, grp = d.a0, s = d.a1, T = S.pos + 1;
      const int p0 = s * P.split;
      if (p0 >= T) break;
      const int p1 = min(p0 + P.split, T);
      const float* q = P.q + ((int64_t)l * P.B + b) * P.nq * P.hd + (int64_t)grp * G * P.hd;
      float* out = P.attn_part + ((((int64_t)l * P.B + b) * P.nkv + grp) * P.nsplit + s) * G * (P.hd + 2);
      const uint16_t* kc = P.kcache + kv_off(P, l, b, grp, 0);
      const uint16_t* vc = P.vcache + kv_off(P, l, b, grp, 0);
      if (P.hd == 128) attn_partial<128>(q, kc, vc, P.hd, p0, p1, G, out, scratch, lane);
      else attn_partial<64>(q, kc, vc, P.hd, p0, p1, G, out, scratch, lane);
      break;
    }
    case TT_MERGE: {
      if (!wait()) return false;
      const int G = P.nq / P.nkv, grp = d.a0, T = S.pos + 1;
      const int used = (T + P.split - 1) / P.split;
      const float* part = P.attn_part + (((int64_t)l * P.B + b) * P.nkv + grp) * P.nsplit * G * (P.hd + 2);
      float* out = P.attn_out + ((int64_t)l * P.B + b) * P.nq * P.hd + (int64_t)grp * G * P.hd;
      if (P.hd == 128) attn_merge<128>(part, used, G, out, lane);
      else attn_merge<64>(part, used, G, out, lane);
      break;
    }
    case TT_ARGMAX: {
      if (!wait()) return false;
      for (int bb = 0; bb < P.B; ++bb) {
        const unsigned long long k =
            __hip_atomic_load(&P.lm_part[bb], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) {
          const float v = argmax_key_value(k);
          S.out[bb] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
          if (!(fabsf(v) <= 3.0e38f)) {  // NaN or Inf won
            atomicCAS(&P.status[1], ST_OK, ST_NONFINITE);
          }
          __hip_atomic_store(&P.lm_part[bb], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      break;
    }
    default:
      break;
  }
  return true;
}

// ---------------------------------------------------------------------------
// Persistent megakernel

__device__ __forceinline__ bool global_abort(const Params& P) {
  return __hip_atomic_load(&P.status[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

__device__ void latch_timeout(const Params& P, Lds* L, int cu, const Task& t, uint32_t value, uint32_t need, int lane) {
  if (lane == 0) {
    if (atomicCAS(&P.status[1], ST_OK, ST_TIMEOUT) == ST_OK) {
      P.status[2] = (uint32_t)cu;
      P.status[3] = t.id;
      P.status[4] = t.in_event;
      P.status[5] = value;
      P.status[6] = need;
    }
    __hip_atomic_store(&P.status[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lds_store(&L->abort, 1u);
  }
}

__device__ void scheduler(const Params& P, const Step& S, Lds* L, float* pages, int page_floats, int cu, int lane) {
  const Task* q = P.tasks + P.queue_off[cu];
  const int n = P.queue_off[cu + 1] - P.queue_off[cu];
  uint16_t cur_key[2] = {0, 0};
  uint32_t uses[2] = {0, 0};
  int last_ev = -1;
  uint32_t last_need = 0;
  for (int f = 0; f < n; ++f) {
    const Task d = q[f];
    if (d.in_event != kNone16) {
      const uint32_t need = d.in_count * S.epoch;
      if (!(d.in_event == last_ev && need <= last_need)) {
        const uint64_t t0 = clock_now();
        uint32_t v;
        while ((v = ld_relaxed_agent(&P.events[d.in_event])) < need) {
          if (global_abort(P)) { if (lane == 0) lds_store(&L->abort, 1u); return; }
          if (clock_now() - t0 > P.timeout_ticks) { latch_timeout(P, L, cu, d, v, need, lane); return; }
          __builtin_amdgcn_s_sleep(1);
        }
        fence_acquire_agent();
        last_ev = d.in_event;
        last_need = need;
      }
    }
    if (d.stage) {
      if (cur_key[d.page] != d.stage) {
        const uint64_t t0 = clock_now();
        while (lds_load(&L->page_done[d.page]) < uses[d.page]) {
          if (clock_now() - t0 > P.timeout_ticks) { latch_timeout(P, L, cu, d, 0, 0, lane); return; }
          __builtin_amdgcn_s_sleep(1);
        }
        fence_acquire_wg();
        stage_input(P, S, d.stage, d.batch, pages + d.page * page_floats, lane);
        cur_key[d.page] = d.stage;
      }
      uses[d.page]++;
    }
    fence_release_wg();
    if (lane == 0) lds_store(&L->frontier, (uint32_t)(f + 1));
  }
}

__device__ void worker(const Params& P, const Step& S, Lds* L, const float* pages, int page_floats, float* scratch,
                       int cu, int lane) {
  const Task* q = P.tasks + P.queue_off[cu];
  const int n = P.queue_off[cu + 1] - P.queue_off[cu];
  for (;;) {
    uint32_t t = 0;
    if (lane == 0) t = lds_add(&L->ticket, 1u);
    t = __builtin_amdgcn_readfirstlane(t);
    if ((int)t >= n) break;
    const Task d = q[t];
    bool aborted = false;
    auto wait = [&]() -> bool {
      while (lds_load(&L->frontier) <= t) {
        if (lds_load(&L->abort)) { aborted = true; return false; }
        __builtin_amdgcn_s_sleep(1);
      }
      fence_acquire_wg();
      return true;
    };
    uint64_t t_start = 0;
    if (P.trace) t_start = clock_now();
    const float* page = d.page != kNone8 ? pages + d.page * page_floats : nullptr;
    if (!exec_task(P, S, d, lane, page, scratch, L, wait) || aborted) break;
    if (P.trace && lane == 0 && (int)d.id < P.trace_cap) {
      P.trace[2 * (int64_t)d.id] = ((unsigned long long)cu << 48) | (t_start & 0xFFFFFFFFFFFFull);
      P.trace[2 * (int64_t)d.id + 1] = clock_now();
    }
    if (d.page != kNone8) {
      fence_release_wg();
      if (lane == 0) lds_add(&L->page_done[d.page], 1u);
    }
    if (d.out_event != kNone16) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores have reached L2
      fence_release_wg();
      uint32_t old = 0;
      if (lane == 0) old = lds_add(&L->slot[d.local_slot], 1u);
      old = __builtin_amdgcn_readfirstlane(old);
      if (old + 1 == d.local_count) {
        if (lane == 0) lds_store(&L->slot[d.local_slot], 0u);
        fence_acq_rel_agent();
        if (d.type == TT_LM && lane == 0) {
          const unsigned long long best =
              __hip_atomic_load(&L->lm_best[d.batch], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          __hip_atomic_fetch_max(&P.lm_part[d.batch], best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&L->lm_best[d.batch], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        fence_acq_rel_agent();
        if (lane == 0) __hip_atomic_fetch_add(&P.events[d.out_event], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

extern "C" __global__ __launch_bounds__(kWaves * kWave, 1) void mk_persistent(Params P, Step S, int page_floats,
                                                                                int scratch_floats) {
  extern __shared__ __align__(16) unsigned char smem[];
  Lds* L = reinterpret_cast<Lds*>(smem);
  float* pages = reinterpret_cast<float*>(smem + sizeof(Lds));
  float* scr = pages + 2 * page_floats;
  const int cu = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (threadIdx.x < kLocalSlots) L->slot[threadIdx.x] = 0;
  if (threadIdx.x < kMaxBatch) L->lm_best[threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    L->frontier = 0;
    L->ticket = 0;
    L->abort = global_abort(P) ? 1u : 0u;
    L->page_done[0] = L->page_done[1] = 0;
  }
  __syncthreads();
  if (L->abort) return;
  if (wave == 0) scheduler(P, S, L, pages, page_floats, cu, lane);
  else worker(P, S, L, pages, page_floats, scr + (wave - 1) * scratch_floats, cu, lane);
}

// ---------------------------------------------------------------------------
// Kernel-per-operator baseline: one launch per stage, the same bodies.
extern "C" __global__ __launch_bounds__(kWaves * kWave) void mk_stage(Params P, Step S, const Task* tasks, int count,
                                                                        int page_floats, int scratch_floats) {
  extern __shared__ __align__(16) unsigned char smem[];
  Lds* L = reinterpret_cast<Lds*>(smem);
  float* page = reinterpret_cast<float*>(smem + sizeof(Lds));
  float* scr = page + page_floats;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (threadIdx.x < kMaxBatch) L->lm_best[threadIdx.x] = 0;
  const Task first = tasks[0];
  if (first.stage && wave == 0) stage_input(P, S, first.stage, first.batch, page, lane);
  __syncthreads();
  auto nowait = []() { return true; };
  for (int i = blockIdx.x * kWaves + wave; i < count; i += gridDim.x * kWaves) {
    Task d = tasks[i];
    exec_task(P, S, d, lane, first.stage ? page : nullptr, scr + wave * scratch_floats, L, nowait);
  }
  if (first.type == TT_LM) {
    __syncthreads();
    if (threadIdx.x < P.B)
      __hip_atomic_fetch_max(&P.lm_part[threadIdx.x], L->lm_best[threadIdx.x], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Fill with a constant bit pattern (poisoning scratch between steps).
extern "C" __global__ void mk_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// ---------------------------------------------------------------------------
// Single-body kernels for unit tests.

// y = W x for W [N, K] bf16; one wave per kRows rows, x staged per workgroup.
extern "C" __global__ __launch_bounds__(kWaves * kWave) void mk_t_gemv_kernel(const uint16_t* W, const float* x,
                                                                                float* y, int N, int K) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* xs = reinterpret_cast<float*>(smem);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave == 0) stage_vector(xs, x, nullptr, K, nullptr, 0.f, lane);
  __syncthreads();
  for (int r0 = (blockIdx.x * kWaves + wave) * kRows; r0 < N; r0 += gridDim.x * kWaves * kRows) {
    GemvRows g;
    g.mask = 0;
    for (int j = 0; j < kRows; ++j) {
      g.row[j] = reinterpret_cast<const v4u*>(W + (int64_t)(r0 + j) * K);
      if (r0 + j < N) g.mask |= 1u << j;
    }
    g.nvec = K / 8;
    v4u buf[kDepth][kRows];
    gemv_prefetch(buf, g, lane);
    float v[kRows];
    gemv_run(buf, g, xs, lane, v);
    if (lane < kRows && r0 + lane < N) y[r0 + lane] = pick4(v, lane);
  }
}

extern "C" __global__ void mk_t_rmsnorm_kernel(const float* x, const uint16_t* gamma, float eps, float* y, int n) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* xs = reinterpret_cast<float*>(smem);
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < kWave) stage_vector(xs, x, nullptr, n, gamma, eps, lane);
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) y[i] = xs[i];
}

// Split-KV attention partials: block = one wave per (group, split).
extern "C" __global__ void mk_t_attn_partial_kernel(const float* q, const uint16_t* k, const uint16_t* v,
                                                    int64_t head_stride, int nq, int nkv, int hd, int T, int split,
                                                    int nsplit, float* part) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* scr = reinterpret_cast<float*>(smem);
  const int grp = blockIdx.x / nsplit, s = blockIdx.x % nsplit, lane = threadIdx.x;
  const int G = nq / nkv, p0 = s * split;
  if (p0 >= T) return;
  const int p1 = min(p0 + split, T);
  float* out = part + ((int64_t)grp * nsplit + s) * G * (hd + 2);
  if (hd == 128)
    attn_partial<128>(q + (int64_t)grp * G * hd, k + grp * head_stride, v + grp * head_stride, hd, p0, p1, G, out, scr, lane);
  else
    attn_partial<64>(q + (int64_t)grp * G * hd, k + grp * head_stride, v + grp * head_stride, hd, p0, p1, G, out, scr, lane);
}

extern "C" __global__ void mk_t_attn_merge_kernel(const float* part, int nq, int nkv, int hd, int T, int split,
                                                  int nsplit, float* o) {
  const int grp = blockIdx.x, lane = threadIdx.x, G = nq / nkv;
  const int used = (T + split - 1) / split;
  const float* p = part + (int64_t)grp * nsplit * G * (hd + 2);
  if (hd == 128) attn_merge<128>(p, used, G, o + (int64_t)grp * G * hd, lane);
  else attn_merge<64>(p, used, G, o + (int64_t)grp * G * hd, lane);
}

// Argmax over fp32 values with the LM-head reduction path: per-wave keys,
// LDS max per workgroup, then a global 64-bit atomic max.
extern "C" __global__ void mk_t_argmax_kernel(const float* x, int n, unsigned long long* slot) {
  __shared__ unsigned long long best;
  if (threadIdx.x == 0) best = 0;
  __syncthreads();
  unsigned long long k = 0;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const unsigned long long c = argmax_key(x[i], (uint32_t)i);
    k = c > k ? c : k;
  }
  k = wave_max_u64(k);
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_max(&best, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_max(slot, best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

extern "C" __global__ void mk_t_argmax_final(const unsigned long long* slot, int32_t* out) {
  if (threadIdx.x == 0) out[0] = (int32_t)(0xFFFFFFFFu - (uint32_t)slot[0]);
}

}  // namespace mk
