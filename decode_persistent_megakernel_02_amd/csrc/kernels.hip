// Device entry points of the kernel-per-operator baseline and the single-body
// test kernels.  The baseline runs one launch per operator over that
// operator's tasks, with the same GEMV task bodies (device.h) as the
// persistent megakernel (mega.hip): every operator's weight rows are cut into
// tasks of R rows, the tasks of one XCD's workgroups are one contiguous part
// of the operator, and inside a workgroup the waves take tasks from an LDS
// counter.  A step is one HIP graph of these launches.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace mk {

// Where a staged input vector comes from.
struct StageSrc {
  const float* f32;   // fp32 source, or
  const uint16_t* bf; // bf16 source (the embedding row of layer 0)
  const uint16_t* gamma;  // RMSNorm gain, null = copy only
  int n;
};

// The RMSNorm gain of a staged input (null: copied without normalising),
// from the per-layer tables.
__device__ __forceinline__ const uint16_t* stage_gain(const Params& P, uint16_t key) {
  switch (stage_kind(key)) {
    case SK_ATTN_NORM: return ld_const(P.attn_norm + stage_layer(key));
    case SK_FFN_NORM: return ld_const(P.ffn_norm + stage_layer(key));
    case SK_FINAL_NORM: return P.final_norm;
    default: return nullptr;
  }
}

__device__ __forceinline__ StageSrc stage_src(const Params& P, const Step& S, uint16_t key, int b,
                                              const uint16_t* gain) {
  const int kind = stage_kind(key), l = stage_layer(key);
  const int64_t H = P.H;
  StageSrc r{nullptr, nullptr, gain, P.H};
  switch (kind) {
    case SK_ATTN_NORM:
      if (l == 0) r.bf = P.embed + (int64_t)token_of(P, S, b) * H;
      else r.f32 = P.xs + ((int64_t)l * P.B + b) * H;
      break;
    case SK_O_IN:
      r.n = P.nq * P.hd;
      r.f32 = P.attn_out + ((int64_t)l * P.B + b) * r.n;
      break;
    case SK_FFN_NORM:
      r.f32 = P.xmid + ((int64_t)l * P.B + b) * H;
      break;
    case SK_H:
      r.n = P.F;
      r.f32 = P.h + ((int64_t)l * P.B + b) * P.F;
      break;
    default:
      r.f32 = P.xs + ((int64_t)P.L * P.B + b) * H;
      break;
  }
  return r;
}

// All kWaves waves of a workgroup stage the vector, in two halves so that
// the loads can be issued before a task's weight prefetch (loads return in
// issue order; staging loads issued after the prefetch would wait for it).
// Each lane owns 8-element groups g = wave*64 + lane + u*512; the first SU
// groups of every lane are loaded by stage_issue into registers, the rest (only
// for vectors longer than SU * 4096) by stage_finish itself.  stage_finish sums
// the squares per wave, then across the waves in a fixed order, normalises,
// and ends with a workgroup barrier; every wave must call it once.
template <int SU>
struct StageRegs {
  v4u raw[SU][2];  // fp32 source: the 8 values; bf16 source: raw[u][0] holds them
  v4u gain[SU];    // the 8 RMSNorm gains (if any)
};

template <int SU>
__device__ __forceinline__ void stage_issue(const StageSrc& r, int wave, int lane, StageRegs<SU>& st) {
  constexpr int NG = kWaves * kWave;
  const int g0 = wave * kWave + lane;
#pragma unroll
  for (int u = 0; u < SU; ++u) {
    const int i = min((g0 + u * NG) * 8, r.n - 8);  // clamped: never predicated (see gemv_run)
    const v4u* a = r.bf ? reinterpret_cast<const v4u*>(r.bf + i) : reinterpret_cast<const v4u*>(r.f32 + i);
    const v4u* b = r.bf ? a : reinterpret_cast<const v4u*>(r.f32 + i + 4);
    st.raw[u][0] = ld_g(a);
    st.raw[u][1] = ld_g(b);
    st.gain[u] = ld_g(r.gamma ? reinterpret_cast<const v4u*>(r.gamma + i) : a);  // no gain: a harmless reload
  }
}

__device__ __forceinline__ void stage_unpack(const StageSrc& r, const v4u& a, const v4u& b, float (&v)[8]) {
  if (r.bf) {
    v[0] = bf_lo(a.x); v[1] = bf_hi(a.x); v[2] = bf_lo(a.y); v[3] = bf_hi(a.y);
    v[4] = bf_lo(a.z); v[5] = bf_hi(a.z); v[6] = bf_lo(a.w); v[7] = bf_hi(a.w);
  } else {
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
}

template <int SU>
__device__ void stage_finish(const Params& P, const StageSrc& r, const StageRegs<SU>& st, float* page, float* red,
                             int wave, int lane) {
  constexpr int NG = kWaves * kWave;
  const int g0 = wave * kWave + lane;
  float ss = 0.f;
  auto put = [&](int i, const float (&v)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
    *reinterpret_cast<float4*>(page + i) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(page + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
  };
#pragma unroll
  for (int u = 0; u < SU; ++u) {
    const int i = (g0 + u * NG) * 8;
    if (i < r.n) {
      float v[8];
      stage_unpack(r, st.raw[u][0], st.raw[u][1], v);
      put(i, v);
    }
  }
  for (int i = (g0 + SU * NG) * 8; i < r.n; i += NG * 8) {  // long vectors only
    const v4u* a = r.bf ? reinterpret_cast<const v4u*>(r.bf + i) : reinterpret_cast<const v4u*>(r.f32 + i);
    const v4u* b = r.bf ? a : reinterpret_cast<const v4u*>(r.f32 + i + 4);
    float v[8];
    stage_unpack(r, ld_g(a), ld_g(b), v);
    put(i, v);
  }
  if (r.gamma) {
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += red[w];
    const float inv = 1.0f / sqrtf(tot / (float)r.n + P.eps);
    for (int i = g0 * 8, u = 0; i < r.n; i += NG * 8, ++u) {  // the groups this lane wrote
      v4u gu = st.gain[0];
#pragma unroll
      for (int k = 1; k < SU; ++k) gu = u == k ? st.gain[k] : gu;
      if (u >= SU) gu = ld_g(reinterpret_cast<const v4u*>(r.gamma + i));
      float4 a = *reinterpret_cast<float4*>(page + i);
      float4 c = *reinterpret_cast<float4*>(page + i + 4);
      a.x = a.x * inv * bf_lo(gu.x); a.y = a.y * inv * bf_hi(gu.x);
      a.z = a.z * inv * bf_lo(gu.y); a.w = a.w * inv * bf_hi(gu.y);
      c.x = c.x * inv * bf_lo(gu.z); c.y = c.y * inv * bf_hi(gu.z);
      c.z = c.z * inv * bf_lo(gu.w); c.w = c.w * inv * bf_hi(gu.w);
      *reinterpret_cast<float4*>(page + i) = a;
      *reinterpret_cast<float4*>(page + i + 4) = c;
    }
  }
  __syncthreads();
}

// The O-projection's input merged straight from the attention split records
// of layer l (batch row 0), when no merge launch runs: for each 8-element
// group of this lane, M = the largest split maximum, weights exp(m_s - M),
// output = sum_s w_s o_s / sum_s w_s l_s (the log-sum-exp merge).  Eight
// splits' maxima, then four splits' records, are loaded per round; every
// load reads a clamped, in-bounds split (weight 0 past the used ones).
// (A one-pass version with a running maximum and eight records per round
// measured no faster and needs 60 more registers.)  Workgroup 0 also stores
// the merged vector as the attention output.  Ends with a workgroup barrier;
// every wave calls it once.
__device__ void stage_merged(const Params& P, const Step& S, int l, float* page, int wave, int lane) {
  const int hd = P.hd, G = P.nq / P.nkv, n = P.nq * hd;
  const int used = (S.pos + 1 + P.split - 1) / P.split;
  const int64_t rs = (int64_t)G * (hd + 2);  // floats between the records of consecutive splits
  constexpr int NG = kWaves * kWave;
  float* out = P.attn_out + (int64_t)l * P.B * n;
  for (int i = (wave * kWave + lane) * 8; i < n; i += NG * 8) {
    const int hq = i / hd, d = i % hd;
    const float* rec = P.attn_part + ((int64_t)l * P.B * P.nkv + hq / G) * P.nsplit * rs + (hq % G) * (hd + 2);
    float M = -INFINITY;
    for (int s0 = 0; s0 < used; s0 += 8) {
      float2 ml[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        ml[k] = *reinterpret_cast<const float2*>(rec + (int64_t)min(s0 + k, used - 1) * rs + hd);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (s0 + k < used && ml[k].y > 0.f) M = fmaxf(M, ml[k].x);
    }
    float L = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    for (int s0 = 0; s0 < used; s0 += 4) {
      float2 ml[4];
      float4 a[4], c[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float* r = rec + (int64_t)min(s0 + k, used - 1) * rs;
        ml[k] = *reinterpret_cast<const float2*>(r + hd);
        a[k] = *reinterpret_cast<const float4*>(r + d);
        c[k] = *reinterpret_cast<const float4*>(r + d + 4);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float w = s0 + k < used && ml[k].y > 0.f ? __expf(ml[k].x - M) : 0.f;
        L = fmaf(w, ml[k].y, L);
        o[0] = fmaf(w, a[k].x, o[0]); o[1] = fmaf(w, a[k].y, o[1]);
        o[2] = fmaf(w, a[k].z, o[2]); o[3] = fmaf(w, a[k].w, o[3]);
        o[4] = fmaf(w, c[k].x, o[4]); o[5] = fmaf(w, c[k].y, o[5]);
        o[6] = fmaf(w, c[k].z, o[6]); o[7] = fmaf(w, c[k].w, o[7]);
      }
    }
    const float inv = 1.0f / L;
    const float4 v0 = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    const float4 v1 = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
    *reinterpret_cast<float4*>(page + i) = v0;
    *reinterpret_cast<float4*>(page + i + 4) = v1;
    if (blockIdx.x == 0) {
      *reinterpret_cast<float4*>(out + i) = v0;
      *reinterpret_cast<float4*>(out + i + 4) = v1;
    }
  }
  __syncthreads();
}

// Rows of a task, with the matrices from the launch arguments.
template <int TT>
__device__ __forceinline__ void gemv_setup(const Params& P, const OpArgs& A, const Task& d,
                                           GemvRows<TaskShape<TT>::R>& g) {
  const uint16_t* W0 = A.w[0];
  if constexpr (TT == TT_QKV) W0 = d.a0 == 0 ? A.w[0] : d.a0 == 1 ? A.w[1] : A.w[2];
  gemv_setup_w<TT>(P, d, W0, A.w[1], g);
}

// Task t of a per-operator launch.
template <int TT>
__device__ __forceinline__ Task op_task(const Params& P, const OpArgs& A, int t) {
  return op_task_fields(TT, A.layer, t, P.H, P.nq, P.nkv, P.hd, P.F, P.V, P.L);
}

// A wave's GEMV tasks with two buffers: the next task's first D chunks are in
// flight while the current task is consumed, so the wave's weight stream
// does not drain between tasks.  The tasks of a workgroup form a pool (slot p
// is task slot_task(p)) whose first 2 * kWaves slots are the waves' first two
// tasks (wave w: slots w and kWaves + w, passed in as i0 and i1); after that,
// and only after the staging barrier that orders the counter's
// initialisation before its first use, a wave takes the next free slot from
// an LDS counter, so a wave that streams faster takes more tasks and the
// workgroup's waves finish together.  (A
// device-wide counter would also balance across CUs, but thousands of waves
// contending on one device-scope atomic serialise at the memory side; it made
// every launch several times slower.)  The R dot products of the wave's j-th
// task go to res[j * R ...] and its index to ids[j] (LDS); the epilogues run
// afterwards (gemv_finish), so that no global store is pending while weight
// loads are in flight (stores and loads share one counter, and a mix of both
// forces a wait for everything).  Returns the number of tasks the wave ran.
template <int TT, bool EXACT, class Wait>
__device__ __forceinline__ int gemv_stream(const Params& P, const OpArgs& A, int count, int i0, int i1, int lane,
                                           const float* page, float* res, int* ids, uint32_t* pool, Wait wait) {
  constexpr int R = TaskShape<TT>::R, D = TaskShape<TT>::D;
  if (i0 >= count) return 0;
  v4u bufA[D][R], bufB[D][R];
  GemvRows<R> gA, gB;
  // Both buffers are filled before the wait for the staged input, so two
  // tasks' weights stream in while the input vector is loaded and normalised.
  gemv_setup<TT>(P, A, op_task<TT>(P, A, i0), gA);
  gemv_prefetch<R, D, EXACT>(bufA, gA, lane);
  float y[R];
  int a = i0, b = i1, j = 0;
  if (b >= count) {
    wait();
    gemv_run<R, D, EXACT>(bufA, gA, page, lane, y);
    gemv_put<TT>(res, ids, j++, a, y, lane);
    return j;
  }
  gemv_setup<TT>(P, A, op_task<TT>(P, A, b), gB);
  gemv_prefetch<R, D, EXACT>(bufB, gB, lane);
  wait();
  for (;;) {  // tasks a (buffer A) and b (buffer B) in flight
    gemv_run<R, D, EXACT>(bufA, gA, page, lane, y);
    gemv_put<TT>(res, ids, j++, a, y, lane);
    a = gemv_next(pool, j, count, lane);
    if (a >= count) {
      gemv_run<R, D, EXACT>(bufB, gB, page, lane, y);
      gemv_put<TT>(res, ids, j++, b, y, lane);
      break;
    }
    gemv_setup<TT>(P, A, op_task<TT>(P, A, a), gA);
    gemv_prefetch<R, D, EXACT>(bufA, gA, lane);
    gemv_run<R, D, EXACT>(bufB, gB, page, lane, y);
    gemv_put<TT>(res, ids, j++, b, y, lane);
    b = gemv_next(pool, j, count, lane);
    if (b >= count) {
      gemv_run<R, D, EXACT>(bufA, gA, page, lane, y);
      gemv_put<TT>(res, ids, j++, a, y, lane);
      break;
    }
    gemv_setup<TT>(P, A, op_task<TT>(P, A, b), gB);
    gemv_prefetch<R, D, EXACT>(bufB, gB, lane);
  }
  return j;
}

// One task's whole epilogue in one lane (the per-operator kernels run the
// epilogues of a wave's tasks side by side, lane j finishing task j).
// Rows as in gemv_setup; y[r] = dot product of row slot r.
template <int TT>
__device__ __forceinline__ void epilogue_lane(const Params& P, const Step& S, const Task& d,
                                              const float (&y)[TaskShape<TT>::R], unsigned long long& best) {
  constexpr int R = TaskShape<TT>::R;
  const int l = d.layer, b = d.batch;
  const int64_t H = P.H;
  if constexpr (TT == TT_QKV) {
    if (d.a3) {  // rotate the pair (lo, hi) = (y0, y1) by the position's angle
      const int half = P.hd / 2, i = d.a1 % P.hd;
      const float c = P.rope_cos[(int64_t)S.pos * half + i], sn = P.rope_sin[(int64_t)S.pos * half + i];
      const float lo = y[0] * c - y[1] * sn, hi = y[1] * c + y[0] * sn;
      if (d.a0 == 0) {
        float* q = P.q + ((int64_t)l * P.B + b) * P.nq * P.hd;
        q[d.a1] = lo;
        q[d.a1 + d.a3] = hi;
      } else {
        const int64_t o = kv_off(P, l, b, d.a1 / P.hd, S.pos);
        kv_store(P, P.kcache, o + i, lo);
        kv_store(P, P.kcache, o + i + half, hi);
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (r < d.a2) {
          const int row = d.a1 + r;
          kv_store(P, P.vcache, kv_off(P, l, b, row / P.hd, S.pos) + row % P.hd, y[r]);
        }
    }
  } else if constexpr (TT == TT_O) {
    const int64_t tok = l == 0 ? (int64_t)token_of(P, S, b) * H : 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < d.a2) {
        const int row = d.a1 + r;
        const float xin = l == 0 ? bf1(P.embed[tok + row]) : P.xs[((int64_t)l * P.B + b) * H + row];
        P.xmid[((int64_t)l * P.B + b) * H + row] = xin + y[r];
      }
  } else if constexpr (TT == TT_GU) {
#pragma unroll
    for (int r = 0; r < R / 2; ++r)
      if (r < d.a2) P.h[((int64_t)l * P.B + b) * P.F + d.a1 + r] = silu(y[r]) * y[r + R / 2];
  } else if constexpr (TT == TT_DOWN) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < d.a2) {
        const int row = d.a1 + r;
        P.xs[((int64_t)(l + 1) * P.B + b) * H + row] = P.xmid[((int64_t)l * P.B + b) * H + row] + y[r];
      }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < d.a2) {
        const int row = d.a1 + r;
        if (S.logits) S.logits[(int64_t)b * P.V + row] = y[r];
        const unsigned long long k = argmax_key(y[r], (uint32_t)row);
        best = k > best ? k : best;
      }
  }
}

// Debug path of the per-operator kernels: a task's raw dot products, at their
// rows of the operator's matrix (QKV: [Wq; Wk; Wv], gate/up: [Wgate; Wup]).
template <int TT>
__device__ __forceinline__ void raw_lane(const Params& P, const Task& d, const float (&y)[TaskShape<TT>::R]) {
  constexpr int R = TaskShape<TT>::R;
  float* o = P.raw_out;
  if constexpr (TT == TT_QKV) {
    const int base = d.a0 == 0 ? 0 : d.a0 == 1 ? P.nq * P.hd : (P.nq + P.nkv) * P.hd;
    if (d.a3) {
      o[base + d.a1] = y[0];
      o[base + d.a1 + d.a3] = y[1];
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (r < d.a2) o[base + d.a1 + r] = y[r];
    }
  } else if constexpr (TT == TT_GU) {
#pragma unroll
    for (int r = 0; r < R / 2; ++r)
      if (r < d.a2) {
        o[d.a1 + r] = y[r];
        o[P.F + d.a1 + r] = y[r + R / 2];
      }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < d.a2) o[d.a1 + r] = y[r];
  }
}

// The epilogues of a wave's n (<= 64) streamed tasks, from their results in
// res and their task indices in ids: lane j finishes task j.
template <int TT>
__device__ __forceinline__ void gemv_finish(const Params& P, const Step& S, const OpArgs& A, int n, int lane,
                                            const float* res, const int* ids, Lds* L) {
  constexpr int R = TaskShape<TT>::R;
  __builtin_amdgcn_wave_barrier();
  unsigned long long best = 0;
  if (lane < n) {
    const Task d = op_task<TT>(P, A, ids[lane]);
    float y[R];
#pragma unroll
    for (int r = 0; r < R; ++r) y[r] = res[lane * R + r];
    if (P.raw_out) raw_lane<TT>(P, d, y);
    else epilogue_lane<TT>(P, S, d, y, best);
  }
  if constexpr (TT == TT_LM) {
    best = wave_max_u64(best);
    if (lane == 0 && n > 0) __hip_atomic_fetch_max(&L->lm_best[0], best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// ---------------------------------------------------------------------------
// Kernel-per-operator path: one launch per operator over that operator's
// tasks, the same bodies.  Wave 0 of each workgroup stages the operator's
// input vector (with its RMSNorm) into LDS once; every wave then takes tasks
// in a workgroup-strided loop.
template <int TT, bool EXACT>
__device__ __forceinline__ void op_body(const Params& P, const Step* Sd, const OpArgs& A, int page_floats,
                                        int scratch_floats) {
  const int count = A.count;
  extern __shared__ __align__(16) unsigned char smem[];
  Lds* L = reinterpret_cast<Lds*>(smem);
  float* page = reinterpret_cast<float*>(smem + sizeof(Lds));
  float* scr = page + page_floats;
  const Step S = ld_const(Sd);
  // wave index made explicitly uniform: task fields are then scalar values
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (threadIdx.x < kMaxBatch) L->lm_best[threadIdx.x] = 0;
  if (threadIdx.x == 0) L->ticket = 2 * kWaves;  // task pool: the first 2 * kWaves slots are the waves' own
  const Task first = op_task<TT>(P, A, 0);
  // Every wave stages its slice of the input vector and passes the staging
  // barriers exactly once: the loads are issued first, then (in gemv_stream)
  // the first task's weight prefetch, then wait() finishes the staging -- or
  // after the loop if the wave has no task.
  constexpr int SU = TT == TT_DOWN ? 4 : 2;  // register-staged groups per lane: vectors up to SU * 4096
  StageSrc src{};
  StageRegs<SU> st;
  const bool merged = TT == TT_O && A.merge && !P.raw_out;  // input merged from the attention splits
  if (first.stage && !merged) {
    if (P.raw_out) {
      // debug: the raw input, copied without normalising.  stage_src is not
      // called here: for layer 0 it reads the step's token, and a raw launch
      // may come before any step has set one.
      src = StageSrc{P.raw_in, nullptr, nullptr,
                     TT == TT_O ? P.nq * P.hd : TT == TT_DOWN ? P.F : P.H};
    } else {
      src = stage_src(P, S, first.stage, first.batch, A.gain);
    }
    stage_issue<SU>(src, wave, lane, st);
  }
  bool staged = false;
  float* red = reinterpret_cast<float*>(L->slot);  // per-wave partial sums of squares
  auto wait = [&]() __attribute__((always_inline)) -> bool {
    if (!staged) {
      if (merged) stage_merged(P, S, A.layer, page, wave, lane);
      else if (first.stage) stage_finish<SU>(P, src, st, page, red, wave, lane);
      else __syncthreads();
      staged = true;
    }
    return true;
  };
  if constexpr (TT == TT_QKV || TT == TT_O || TT == TT_GU || TT == TT_DOWN || TT == TT_LM) {
    // scratch_floats = result slots per wave (R per task of this wave)
    const int i0 = slot_task(wave, count), i1 = slot_task(kWaves + wave, count), wid = blockIdx.x * kWaves + wave;
    float* res = scr + wave * scratch_floats;
    int* ids = reinterpret_cast<int*>(res + kMaxTasksPerWave * TaskShape<TT>::R);
    // optional wave timeline (debug): start, input staged, stream done, epilogues done
    const bool tr = P.trace && P.trace_op == ((TT << 16) | first.layer) && 4 * (wid + 1) <= 2 * P.trace_cap;
    const uint64_t t0 = tr ? clock_now() : 0;
    uint64_t t1 = 0;
    auto wait_tr = [&]() __attribute__((always_inline)) -> bool {
      const bool r = wait();
      if (tr && !t1) t1 = clock_now();
      return r;
    };
    const int n = gemv_stream<TT, EXACT>(P, A, count, i0, i1, lane, page, res, ids, &L->ticket, wait_tr);
    const uint64_t t2 = tr ? clock_now() : 0;
    wait();
    gemv_finish<TT>(P, S, A, n, lane, res, ids, L);
    if (tr && lane == 0) {
      const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID: wave, SIMD, CU, SE
      const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20);  // XCC_ID
      unsigned long long* o = P.trace + 4 * (int64_t)wid;
      o[0] = ((unsigned long long)((xcc & 0xF) << 28 | (hw & 0x0FFFFFFF)) << 32) | (uint32_t)t0;
      o[1] = t1;
      o[2] = t2;
      o[3] = clock_now();
    }
  } else {
    static_assert(TT == TT_ARGMAX, "per-operator kernels: GEMV operators and the argmax");
    // the LM head's running keys -> greedy ids; the keys are cleared for the next step
    if (blockIdx.x == 0 && wave == 0 && lane == 0) {
      for (int bb = 0; bb < P.B; ++bb) {
        const unsigned long long k = __hip_atomic_load(&P.lm_part[bb], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        S.out[bb] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
        if (!(fabsf(argmax_key_value(k)) <= 3.0e38f)) atomicCAS(&P.status[1], ST_OK, ST_NONFINITE);  // NaN or Inf won
        __hip_atomic_store(&P.lm_part[bb], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  wait();
  if constexpr (TT == TT_LM) {
    __syncthreads();
    if (threadIdx.x < P.B && !P.raw_out)
      __hip_atomic_fetch_max(&P.lm_part[threadIdx.x], L->lm_best[threadIdx.x], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Each GEMV operator has a generic kernel and an _x kernel for K a multiple of
// 512 whose chunk count is a multiple of D (no clamped loads).
#define MK_OP_KERNEL(name, TT, EXACT)                                                                      \
  extern "C" __global__ __launch_bounds__(kWaves * kWave) void name(Params P, const Step* S, OpArgs A, int pf, \
                                                                      int sf) {                            \
    op_body<TT, EXACT>(P, S, A, pf, sf);                                                                   \
  }
MK_OP_KERNEL(mk_op_qkv, TT_QKV, false)
MK_OP_KERNEL(mk_op_o, TT_O, false)
MK_OP_KERNEL(mk_op_gu, TT_GU, false)
MK_OP_KERNEL(mk_op_down, TT_DOWN, false)
MK_OP_KERNEL(mk_op_lm, TT_LM, false)
MK_OP_KERNEL(mk_op_argmax, TT_ARGMAX, false)
MK_OP_KERNEL(mk_op_qkv_x, TT_QKV, true)
MK_OP_KERNEL(mk_op_o_x, TT_O, true)
MK_OP_KERNEL(mk_op_gu_x, TT_GU, true)
MK_OP_KERNEL(mk_op_down_x, TT_DOWN, true)
MK_OP_KERNEL(mk_op_lm_x, TT_LM, true)

// Attention, per-operator path: one workgroup of NW waves per (batch row, KV
// group, split).  The split's positions are dealt to the waves in blocks;
// each wave keeps an online-softmax state; the workgroup merges its waves'
// states through LDS.  With a single split (FINAL) the result is normalised
// and written as the attention output itself (and, on the batched path, the
// O-projection's operand planes), so no merge launch follows; otherwise it
// is one (o, m, l) record per head for the merge.
template <int HD, typename KT, int NW, bool FINAL, int GQ>
__device__ __forceinline__ void attn_split_wg(const Params& P, const Step& S, int l, int b, int grp, int s, float* sm,
                                              int wave, int lane, uint64_t* stamps) {
  using Gm = AttnGeom<HD, KT>;
  const int G = P.nq / P.nkv, T = S.pos + 1;
  const int p0 = s * P.split, p1 = min(p0 + P.split, T);
  if (p0 >= T) return;
  float* qs = sm;                // [G][HD]
  float* recs = qs + G * HD;     // [NW][G][HD + 2]
  const float* q = P.q + ((int64_t)l * P.B + b) * P.nq * P.hd + (int64_t)grp * G * HD;
  const int64_t o0 = kv_off(P, l, b, grp, 0);
  const KT* kc = static_cast<const KT*>(P.kcache) + o0;
  const KT* vc = static_cast<const KT*>(P.vcache) + o0;
  // The query loads first (every block needs them), then this wave's first
  // K/V block; only then wait for the queries.
  constexpr int QPT = (GqaHeads<GQ>::MAX * HD + NW * kWave - 1) / (NW * kWave);
  float qv[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) qv[i] = q[min((int)threadIdx.x + i * NW * kWave, G * HD - 1)];
  // bf16 cache at head_dim 128: scores on the matrix cores (attn_compute_mf)
  constexpr bool MF = HD == 128 && sizeof(KT) == 2;
  const int b0 = p0 + wave * Gm::NP;
  std::conditional_t<MF, AttnBufMf, AttnBuf<HD, KT>> A, B;
  if (b0 < p1) {
    if constexpr (MF) attn_load_mf(kc, vc, b0, p1, lane, A);
    else attn_load<HD, KT>(kc, vc, b0, p1, lane, A);
  }
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int idx = threadIdx.x + i * NW * kWave;
    if (idx < G * HD) qs[idx] = qv[i];
  }
  __syncthreads();
  if (stamps) stamps[1] = clock_now();
  if constexpr (MF) {
    AttnQFrag qf;
    attn_q_frags(qs, G, lane, qf);
    AttnStateMf st;
    st.init();
    // The wave's record slot (G * 130 floats, an even offset) holds the
    // weights ([G][16], 16-byte aligned) until the records are written.
    static_assert(16 * kMaxGqa + 2 <= HD + 2, "the weights fit the wave's records");
    float* pw = recs + ((wave * G * (HD + 2) + 3) & ~3);
    if (b0 < p1) attn_pipeline_mf(A, B, qf, kc, vc, b0, p1, NW * Gm::NP, G, lane, pw, st);
    if (stamps) stamps[2] = clock_now();
    attn_store_state_mf(st, G, recs + wave * G * (HD + 2), lane);
  } else {
    AttnState<HD, GQ> st;
    st.init();
    if (b0 < p1) attn_pipeline<HD, KT, GQ>(A, B, qs, kc, vc, b0, p1, NW * Gm::NP, G, lane, st);
    if (stamps) stamps[2] = clock_now();
    attn_store_state<HD, GQ>(st, G, recs + wave * G * (HD + 2), lane);
  }
  __syncthreads();
  for (int h = wave; h < G; h += NW) {
    // merge the waves' records of head h
    constexpr int DPL = HD / kWave;
    float M = -INFINITY, Ls = 0.f, o[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = 0.f;
    for (int w = 0; w < NW; ++w) {
      const float* r = recs + (w * G + h) * (HD + 2);
      const float lw = r[HD + 1];
      if (!(lw > 0.f)) continue;
      const float mw = r[HD], Mn = fmaxf(M, mw);
      const float a = __expf(M - Mn), c = __expf(mw - Mn);
      Ls = Ls * a + lw * c;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = o[e] * a + r[lane * DPL + e] * c;
      M = Mn;
    }
    if constexpr (FINAL) {
      const int64_t col = (int64_t)(grp * G + h) * HD + lane * DPL;
      float* out = P.attn_out + ((int64_t)l * P.B + b) * P.nq * P.hd + col;
      const float inv = 1.0f / Ls;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        out[e] = o[e] * inv;
        if (P.ao) {
          uint16_t* hi = P.ao + (int64_t)b * P.nq * P.hd + col + e;
          split_bf16(o[e] * inv, hi, hi + (int64_t)P.Bp * P.nq * P.hd);
        }
      }
    } else {
      float* oh = P.attn_part + ((((int64_t)l * P.B + b) * P.nkv + grp) * P.nsplit + s) * G * (HD + 2) + h * (HD + 2);
#pragma unroll
      for (int e = 0; e < DPL; ++e) oh[lane * DPL + e] = o[e];
      if (lane == 0) {
        oh[HD] = M;
        oh[HD + 1] = Ls;
      }
    }
  }
}

// Log-sum-exp merge of the used splits of (batch row b, KV group grp): query
// head h of the group by wave h % nw.  Writes the fp32 attention output and,
// on the batched path, the O-projection's bf16 operand planes.
__device__ __forceinline__ void merge_group(const Params& P, int layer, int b, int grp, int used, int wave, int nw,
                                            int lane) {
  const int G = P.nq / P.nkv;
  const float* part = P.attn_part + (((int64_t)layer * P.B + b) * P.nkv + grp) * P.nsplit * G * (P.hd + 2);
  for (int h = wave; h < G; h += nw) {
    const int64_t col = (int64_t)(grp * G + h) * P.hd;
    float* out = P.attn_out + ((int64_t)layer * P.B + b) * P.nq * P.hd + col;
    uint16_t* ohi = P.ao ? P.ao + (int64_t)b * P.nq * P.hd + col : nullptr;
    uint16_t* olo = P.ao ? ohi + (int64_t)P.Bp * P.nq * P.hd : nullptr;
    if (P.hd == 128) attn_merge<128>(part + h * (128 + 2), used, 1, out, lane, G * (128 + 2), ohi, olo);
    else attn_merge<64>(part + h * (64 + 2), used, 1, out, lane, G * (64 + 2), ohi, olo);
  }
}

// Optional wave timeline of an attention launch (debug): entry, queries
// staged, positions done, exit -- the layout of the GEMV operator timelines.
struct AttnTrace {
  uint64_t t[4];
  bool on;
  __device__ AttnTrace(const Params& P, int layer, int nwaves) {
    const int wid = blockIdx.x * nwaves + (int)(threadIdx.x >> 6);
    on = P.trace && P.trace_op == ((TT_ATTN << 16) | layer) && 4 * (wid + 1) <= 2 * P.trace_cap;
    t[0] = on ? clock_now() : 0;
    t[1] = t[2] = t[3] = 0;
  }
  __device__ uint64_t* stamps() { return on ? t : nullptr; }
  __device__ void write(const Params& P, int nwaves) {
    if (!on || (threadIdx.x & 63)) return;
    const int wid = blockIdx.x * nwaves + (int)(threadIdx.x >> 6);
    const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
    const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20);
    unsigned long long* o = P.trace + 4 * (int64_t)wid;
    o[0] = ((unsigned long long)((xcc & 0xF) << 28 | (hw & 0x0FFFFFFF)) << 32) | (uint32_t)t[0];
    o[1] = t[1];
    o[2] = t[2];
    o[3] = clock_now();
  }
};

// Split-KV attention, one workgroup per (batch row, KV group, split).  With
// `fuse_merge`, the last workgroup of a (batch row, KV group) to finish
// merges all its splits: every workgroup publishes its records with an
// agent-scope fence and counts itself in attn_count; the one that brings the
// count to the number of used splits acquires, merges, and resets the count
// for the next launch.  No workgroup ever waits for another.  GQ: the query
// heads per KV group when fixed at compile time (0: given at run time).
template <typename KT, int GQ>
__device__ __forceinline__ void attn_split_body(const Params& P, const Step* Sd, int layer, int fuse_merge) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* sm = reinterpret_cast<float*>(smem);
  __shared__ uint32_t is_last;
  const Step S = ld_const(Sd);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s = blockIdx.x % P.nsplit, bg = blockIdx.x / P.nsplit;
  const int b = bg / P.nkv, grp = bg % P.nkv;
  const int used = (S.pos + 1 + P.split - 1) / P.split;
  if (s >= used) return;  // past the current length: no record, not counted
  AttnTrace tr(P, layer, kAttnWaves);
  if (P.hd == 128) attn_split_wg<128, KT, kAttnWaves, false, GQ>(P, S, layer, b, grp, s, sm, wave, lane, tr.stamps());
  else attn_split_wg<64, KT, kAttnWaves, false, GQ>(P, S, layer, b, grp, s, sm, wave, lane, tr.stamps());
  tr.write(P, kAttnWaves);
  if (!fuse_merge) return;
  __threadfence();  // release this wave's records at agent scope
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&P.attn_count[bg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = old + 1 == (uint32_t)used;
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();  // acquire the other workgroups' records
  merge_group(P, layer, b, grp, used, wave, kAttnWaves, lane);
  if (threadIdx.x == 0) __hip_atomic_store(&P.attn_count[bg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Whole-context attention: one workgroup of kAttnFullWaves waves per (batch
// row, KV group) covers every position and writes the final output (used
// when the context fits one split).
template <typename KT, int GQ>
__device__ __forceinline__ void attn_full_body(const Params& P, const Step* Sd, int layer) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* sm = reinterpret_cast<float*>(smem);
  const Step S = ld_const(Sd);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.x / P.nkv, grp = blockIdx.x % P.nkv;
  AttnTrace tr(P, layer, kAttnFullWaves);
  if (P.hd == 128) attn_split_wg<128, KT, kAttnFullWaves, true, GQ>(P, S, layer, b, grp, 0, sm, wave, lane, tr.stamps());
  else attn_split_wg<64, KT, kAttnFullWaves, true, GQ>(P, S, layer, b, grp, 0, sm, wave, lane, tr.stamps());
  tr.write(P, kAttnFullWaves);
}

// One kernel pair per cache element type and group size, so that each gets
// its own register allocation: the state arrays hold exactly the group's
// heads (with room for 8 heads and both element types in one kernel they no
// longer fit in registers and spilled to scratch).  The split kernel asks for
// two waves per SIMD: left free, the compiler gave the matrix-core variant 272
// registers, one wave per SIMD, and the 8-sequence 4K-context attention took
// 39.3 us per layer against 32.3 us with 225 registers.
#define MK_ATTN_KERNELS(KN, KT, GQ)                                                                           \
  extern "C" __global__ __launch_bounds__(kAttnWaves * kWave, 2) void mk_op_attn_split_##KN##_g##GQ(          \
      Params P, const Step* Sd, int layer, int fuse_merge) {                                                  \
    attn_split_body<KT, GQ>(P, Sd, layer, fuse_merge);                                                        \
  }                                                                                                           \
  extern "C" __global__ __launch_bounds__(kAttnFullWaves * kWave) void mk_op_attn_full_##KN##_g##GQ(          \
      Params P, const Step* Sd, int layer) {                                                                  \
    attn_full_body<KT, GQ>(P, Sd, layer);                                                                     \
  }
#define MK_ATTN_KERNELS_G(KN, KT) \
  MK_ATTN_KERNELS(KN, KT, 0) MK_ATTN_KERNELS(KN, KT, 1) MK_ATTN_KERNELS(KN, KT, 2) MK_ATTN_KERNELS(KN, KT, 4) \
  MK_ATTN_KERNELS(KN, KT, 8)
MK_ATTN_KERNELS_G(f32, float)
MK_ATTN_KERNELS_G(bf16, uint16_t)
#undef MK_ATTN_KERNELS_G
#undef MK_ATTN_KERNELS

// Log-sum-exp merge as its own launch: one wave per (batch row, query head).
extern "C" __global__ __launch_bounds__(kMaxGqa * kWave) void mk_op_attn_merge(Params P, const Step* Sd, int layer) {
  const Step S = ld_const(Sd);
  const int G = P.nq / P.nkv, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave >= G) return;
  const int b = blockIdx.x / P.nkv, grp = blockIdx.x % P.nkv;
  const int used = (S.pos + 1 + P.split - 1) / P.split;
  merge_group(P, layer, b, grp, used, wave, G, lane);
}

// Per-step arguments live in device memory so that a step's launches can be
// replayed as one static graph; this kernel writes them.
extern "C" __global__ void mk_set_step(Step* dst, Step s) {
  if (threadIdx.x == 0) *dst = s;
}

// Fill with a constant bit pattern (poisoning scratch between steps).
extern "C" __global__ void mk_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// ---------------------------------------------------------------------------
// Single-body kernels for unit tests.

// y = W x for W [N, K] bf16; one wave per 4 rows (8 chunks deep), x staged per workgroup.
extern "C" __global__ __launch_bounds__(kWaves * kWave) void mk_t_gemv_kernel(const uint16_t* W, const float* x,
                                                                                float* y, int N, int K) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* xs = reinterpret_cast<float*>(smem);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave == 0) stage_vector(xs, x, nullptr, K, nullptr, 0.f, lane);
  __syncthreads();
  constexpr int R = 4, D = 8;
  for (int r0 = (blockIdx.x * kWaves + wave) * R; r0 < N; r0 += gridDim.x * kWaves * R) {
    GemvRows<R> g;
    g.base0 = g.base1 = reinterpret_cast<const v4u*>(W + (int64_t)r0 * K);
    g.stride = K / 8;
    g.split = R;
    g.mask = (1u << min(R, N - r0)) - 1;
    g.nvec = K / 8;
    v4u buf[D][R];
    gemv_prefetch<R, D, false>(buf, g, lane);
    float v[R];
    gemv_run<R, D, false>(buf, g, xs, lane, v);
    if (lane < R && r0 + lane < N) y[r0 + lane] = pick<R>(v, lane);
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
template <typename KT>
__device__ void t_attn_partial(const float* q, const void* k, const void* v, int64_t head_stride, int nq, int nkv,
                               int hd, int T, int split, int nsplit, float* part) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* scr = reinterpret_cast<float*>(smem);
  const int grp = blockIdx.x / nsplit, s = blockIdx.x % nsplit, lane = threadIdx.x;
  const int G = nq / nkv, p0 = s * split;
  if (p0 >= T) return;
  const int p1 = min(p0 + split, T);
  float* out = part + ((int64_t)grp * nsplit + s) * G * (hd + 2);
  const KT* kc = static_cast<const KT*>(k) + grp * head_stride;
  const KT* vc = static_cast<const KT*>(v) + grp * head_stride;
  if (hd == 128) attn_partial<128, KT>(q + (int64_t)grp * G * hd, kc, vc, p0, p1, G, out, scr, lane);
  else attn_partial<64, KT>(q + (int64_t)grp * G * hd, kc, vc, p0, p1, G, out, scr, lane);
}

extern "C" __global__ __launch_bounds__(kWave) void mk_t_attn_partial_kernel(const float* q, const void* k, const void* v, int64_t head_stride,
                                                    int nq, int nkv, int hd, int T, int split, int nsplit, int kv_f32,
                                                    float* part) {
  if (kv_f32) t_attn_partial<float>(q, k, v, head_stride, nq, nkv, hd, T, split, nsplit, part);
  else t_attn_partial<uint16_t>(q, k, v, head_stride, nq, nkv, hd, T, split, nsplit, part);
}

extern "C" __global__ __launch_bounds__(kWave) void mk_t_attn_merge_kernel(const float* part, int nq, int nkv, int hd, int T, int split,
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

// Streaming read of nvec 16-byte vectors (HBM ceiling probe): every thread
// keeps U non-temporal loads in flight; the xor of the data decides a store
// that never happens for a constant-filled buffer, so no load is dead.
template <int U>
__global__ __launch_bounds__(512) void stream_read_kernel(const v4u* src, int64_t nvec, uint32_t* sink) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, nth = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  int64_t i = tid;
  for (; i + (U - 1) * nth < nvec; i += U * nth) {
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld_w(src + i + u * nth);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < nvec; i += nth) {
    const v4u v = ld_w(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* src, int64_t nvec, int wgs, int loads, uint32_t* sink, hipStream_t st) {
  const v4u* p = static_cast<const v4u*>(src);
  if (loads == 4) hipLaunchKernelGGL(stream_read_kernel<4>, dim3(wgs), dim3(512), 0, st, p, nvec, sink);
  else if (loads == 8) hipLaunchKernelGGL(stream_read_kernel<8>, dim3(wgs), dim3(512), 0, st, p, nvec, sink);
  else hipLaunchKernelGGL(stream_read_kernel<16>, dim3(wgs), dim3(512), 0, st, p, nvec, sink);
  return hipGetLastError();
}

extern "C" __global__ void mk_t_argmax_final(const unsigned long long* slot, int32_t* out) {
  if (threadIdx.x == 0) out[0] = (int32_t)(0xFFFFFFFFu - (uint32_t)slot[0]);
}

}  // namespace mk
