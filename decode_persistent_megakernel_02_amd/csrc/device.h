// Device helpers and task bodies shared by the persistent runtime, the
// kernel-per-operator baseline and the single-body test kernels.
//
// Bodies are written for one 64-lane wavefront each: a worker wave owns a task
// from start to end, so no workgroup barrier is ever taken inside a task.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mk_internal.h"

namespace mk {

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (bf16 is the upper half of an fp32 bit pattern)
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf1(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even (finite inputs)
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Cross-lane reductions with DPP inside each 16-lane row, then the four row
// results combined through readlane (uniform result in every lane).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float rd_lane(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  return (rd_lane(v, 0) + rd_lane(v, 16)) + (rd_lane(v, 32) + rd_lane(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(fmaxf(rd_lane(v, 0), rd_lane(v, 16)), fmaxf(rd_lane(v, 32), rd_lane(v, 48)));
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}

// Argmax key: larger key = larger value, ties -> smaller index.
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t idx) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (0xFFFFFFFFu - idx);
}
__device__ __forceinline__ float argmax_key_value(unsigned long long k) {
  uint32_t u = (uint32_t)(k >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------------------
// Memory ordering (HIP scoped atomics; the compiler emits the gfx950 cache
// maintenance for each scope).
__device__ __forceinline__ uint32_t ld_relaxed_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void fence_acq_rel_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent"); }
__device__ __forceinline__ void fence_release_wg() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup"); }
__device__ __forceinline__ void fence_acquire_wg() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup"); }
__device__ __forceinline__ uint32_t lds_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint32_t lds_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint64_t clock_now() { return __builtin_amdgcn_s_memrealtime(); }

// ---------------------------------------------------------------------------
// GEMV core: R weight rows (bf16, each K contiguous elements) dotted with one
// fp32 vector held in LDS.  Each lane owns 8 consecutive columns of every
// 512-column chunk, so one wave load instruction reads 1 KiB of a row.  D
// chunks per row stay in flight (R*D loads of 16 B per lane); `prefetch`
// issues them -- weights depend on no event, so this can run before the
// task's inputs exist -- and `run` consumes them, refilling each slot with the
// chunk D ahead.
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Row r (r < split) starts at base0 + r * stride, row r >= split at
// base1 + (r - split) * stride (both in 16-byte vectors).  With r a
// compile-time constant after unrolling, every address is base + constant.
// A row outside `mask` reads row 0 instead (always in bounds; its result is
// discarded), so no load is ever predicated.
template <int R>
struct GemvRows {
  const v4u* base0;
  const v4u* base1;
  int64_t stride;  // vectors between consecutive rows
  int split;       // rows taken from base0
  uint32_t mask;   // bit r set: row r valid (bit 0 always set)
  int nvec;        // K / 8 (16-byte vectors per row)
  __device__ __forceinline__ const v4u* row(int r) const {
    if (!((mask >> r) & 1)) return base0;
    return r < split ? base0 + r * stride : base1 + (r - split) * stride;
  }
};

// Weight loads go through the global address space explicitly: the layer
// pointer tables hold generic pointers, and a generic (flat) load also counts
// against the LDS counter, so every wait for one weight vector would drain
// all loads in flight.
typedef const __attribute__((address_space(1))) v4u* gv4u_ptr;
__device__ __forceinline__ v4u ld_w(const v4u* p) { return __builtin_nontemporal_load((gv4u_ptr)p); }
__device__ __forceinline__ v4u ld_g(const v4u* p) { return *(gv4u_ptr)p; }

// Every streaming load below is unconditional.  A load under a divergent
// branch leaves the compiler unable to count loads in flight, and it then
// waits for all of them at the next use, draining the pipeline.  With EXACT
// (K a multiple of 512 and the chunk count a multiple of D, true of every
// production shape) no lane is ever out of range and every address is the
// row base plus a constant; otherwise out-of-range vectors read a clamped,
// in-bounds address and are zeroed on the activation side.
template <int R, int D, bool EXACT>
__device__ __forceinline__ void gemv_prefetch(v4u (&buf)[D][R], const GemvRows<R>& g, int lane) {
#pragma unroll
  for (int s = 0; s < D; ++s) {
    const int v = EXACT ? s * kWave + lane : min(s * kWave + lane, g.nvec - 1);
#pragma unroll
    for (int r = 0; r < R; ++r) buf[s][r] = ld_w(g.row(r) + v);
  }
}

__device__ __forceinline__ float dot8(v4u w, const float4& a, const float4& b, float acc) {
  acc = fmaf(bf_lo(w.x), a.x, acc);
  acc = fmaf(bf_hi(w.x), a.y, acc);
  acc = fmaf(bf_lo(w.y), a.z, acc);
  acc = fmaf(bf_hi(w.y), a.w, acc);
  acc = fmaf(bf_lo(w.z), b.x, acc);
  acc = fmaf(bf_hi(w.z), b.y, acc);
  acc = fmaf(bf_lo(w.w), b.z, acc);
  acc = fmaf(bf_hi(w.w), b.w, acc);
  return acc;
}

// Chunk c (vectors c*64 + lane) of the R rows, held in `slot`, dotted with xs.
template <int R, bool EXACT>
__device__ __forceinline__ void gemv_consume(const v4u (&slot)[R], int c, int nvec, const float* xs, int lane,
                                             float (&acc)[R]) {
  const int v = c * kWave + lane, vc = EXACT ? v : min(v, nvec - 1);
  float4 xa = *reinterpret_cast<const float4*>(xs + vc * 8);
  float4 xb = *reinterpret_cast<const float4*>(xs + vc * 8 + 4);
  if (!EXACT && v >= nvec) xa = xb = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = dot8(slot[r], xa, xb, acc[r]);
}

// y[r] = sum_k W[r][k] * xs[k] for the R rows (uniform across the wave).  The
// chunks run in rounds of D: every round but the last refills each slot with
// the chunk D ahead right after consuming it, the last round only consumes.
template <int R, int D, bool EXACT>
__device__ __forceinline__ void gemv_run(v4u (&buf)[D][R], const GemvRows<R>& g, const float* xs, int lane,
                                         float (&y)[R]) {
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  const int nchunks = (g.nvec + kWave - 1) / kWave, nrounds = (nchunks + D - 1) / D;
  for (int rd = 0; rd + 1 < nrounds; ++rd) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int c = rd * D + s;
      gemv_consume<R, EXACT>(buf[s], c, g.nvec, xs, lane, acc);
      const int vn = EXACT ? (c + D) * kWave + lane : min((c + D) * kWave + lane, g.nvec - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) buf[s][r] = ld_w(g.row(r) + vn);
    }
  }
#pragma unroll
  for (int s = 0; s < D; ++s) gemv_consume<R, EXACT>(buf[s], (nrounds - 1) * D + s, g.nvec, xs, lane, acc);
#pragma unroll
  for (int r = 0; r < R; ++r) y[r] = wave_sum(acc[r]);
}

// ---------------------------------------------------------------------------
// Staging: one wave loads an activation vector into an LDS page, applying
// RMSNorm (x * (mean(x^2) + eps)^-1/2 * gamma) when a gain is given.
__device__ __forceinline__ void stage_vector(float* page, const float* src, const uint16_t* src_bf16, int n,
                                             const uint16_t* gamma, float eps, int lane) {
  float ss = 0.f;
  for (int i = lane * 8; i < n; i += kWave * 8) {
    float v[8];
    if (src_bf16) {
      const uint4 u = *reinterpret_cast<const uint4*>(src_bf16 + i);
      v[0] = bf_lo(u.x); v[1] = bf_hi(u.x); v[2] = bf_lo(u.y); v[3] = bf_hi(u.y);
      v[4] = bf_lo(u.z); v[5] = bf_hi(u.z); v[6] = bf_lo(u.w); v[7] = bf_hi(u.w);
    } else {
      const float4 a = *reinterpret_cast<const float4*>(src + i);
      const float4 b = *reinterpret_cast<const float4*>(src + i + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
    *reinterpret_cast<float4*>(page + i) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(page + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  if (gamma) {
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)n + eps);
    for (int i = lane * 8; i < n; i += kWave * 8) {
      const uint4 gu = *reinterpret_cast<const uint4*>(gamma + i);
      float4 a = *reinterpret_cast<float4*>(page + i);
      float4 b = *reinterpret_cast<float4*>(page + i + 4);
      a.x = a.x * inv * bf_lo(gu.x); a.y = a.y * inv * bf_hi(gu.x);
      a.z = a.z * inv * bf_lo(gu.y); a.w = a.w * inv * bf_hi(gu.y);
      b.x = b.x * inv * bf_lo(gu.z); b.y = b.y * inv * bf_hi(gu.z);
      b.z = b.z * inv * bf_lo(gu.w); b.w = b.w * inv * bf_hi(gu.w);
      *reinterpret_cast<float4*>(page + i) = a;
      *reinterpret_cast<float4*>(page + i + 4) = b;
    }
  }
}

// ---------------------------------------------------------------------------
// Split-KV decode attention (online softmax).  One wave owns a running state
// for the G query heads of a KV group: max score m, sum of exp(score - m) l,
// and the unnormalised output o (each lane owns DPL = HD/64 dims).  The cache
// element type KT is bf16 (uint16_t) or fp32 (float).
//
// A block covers NP positions.  For the scores, LPP lanes share one position
// (each lane holds 64 bytes of the K row -- 32 bf16 or 16 fp32 elements --
// loaded with 16-byte loads) and their partial dot products are combined with
// DPP swaps inside the group of LPP lanes.
// For the values, every lane owns DPL dims of every position.  K and V of the
// whole block are loaded up front, so a block costs one memory round trip.
template <int HD, typename KT>
struct AttnGeom {
  static constexpr int EPL = sizeof(KT) == 4 ? 16 : 32;      // K elements per lane (64 bytes)
  static constexpr int LPP = HD / EPL;                        // lanes per position (2, 4 or 8)
  static constexpr int NP = kWave / LPP;                      // positions per block (32, 16 or 8)
  static constexpr int KV16 = EPL * (int)sizeof(KT) / 16;    // 16-byte K loads per lane
  static constexpr int DPL = HD / kWave;                      // V dims per lane
};

// GQ: the query heads per KV group when fixed at compile time (the state and
// score arrays then hold exactly GQ heads), or 0: up to kMaxGqa heads, the
// count given at run time.
template <int GQ>
struct GqaHeads {
  static constexpr int MAX = GQ ? GQ : kMaxGqa;
  __device__ static constexpr bool has(int h, int G) { return GQ ? h < GQ : h < G; }
};

template <int HD, int GQ = 0>
struct AttnState {
  static constexpr int DPL = HD / kWave, GM = GqaHeads<GQ>::MAX;
  float m[GM], l[GM], o[GM][DPL];
  __device__ void init() {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[h][e] = 0.f;
    }
  }
};

// 8 K elements at a 16-byte vector (bf16: one vector; fp32: two vectors).
template <typename KT>
__device__ __forceinline__ float dot_k(const v4u* kv, int i, const float* q, float acc) {
  const float4 a = *reinterpret_cast<const float4*>(q);
  const float4 b = *reinterpret_cast<const float4*>(q + 4);
  if constexpr (sizeof(KT) == 2) {
    return dot8(kv[i], a, b, acc);
  } else {
    const v4u u = kv[2 * i], w = kv[2 * i + 1];
    acc = fmaf(__uint_as_float(u.x), a.x, acc);
    acc = fmaf(__uint_as_float(u.y), a.y, acc);
    acc = fmaf(__uint_as_float(u.z), a.z, acc);
    acc = fmaf(__uint_as_float(u.w), a.w, acc);
    acc = fmaf(__uint_as_float(w.x), b.x, acc);
    acc = fmaf(__uint_as_float(w.y), b.y, acc);
    acc = fmaf(__uint_as_float(w.z), b.z, acc);
    return fmaf(__uint_as_float(w.w), b.w, acc);
  }
}

// A block's K and V in registers: K, this lane's part of its position's row;
// V, this lane's dims of every position of the block.
template <int HD, typename KT>
struct AttnBuf {
  using Gm = AttnGeom<HD, KT>;
  static constexpr int VW = (Gm::DPL * (int)sizeof(KT) + 3) / 4;  // 32-bit words of V per lane and position
  v4u kr[Gm::KV16];
  uint32_t vr[Gm::NP][VW];
};

typedef const __attribute__((address_space(1))) uint32_t* gu32_ptr;
typedef const __attribute__((address_space(1))) uint16_t* gu16_ptr;

// Issues the K loads of the block [p0, p0 + NP).  Positions at or past p1
// read position p1 - 1 (in bounds; attn_compute masks them), so no load is
// predicated.  kc: this group's cache rows (position p at + p * HD).
template <int HD, typename KT>
__device__ __forceinline__ void attn_load_k(const KT* kc, int p0, int p1, int lane, AttnBuf<HD, KT>& bf) {
  using Gm = AttnGeom<HD, KT>;
  const int my = lane / Gm::LPP, part = lane % Gm::LPP;
  const v4u* krow = reinterpret_cast<const v4u*>(kc + (int64_t)min(p0 + my, p1 - 1) * HD + part * Gm::EPL);
#pragma unroll
  for (int i = 0; i < Gm::KV16; ++i) bf.kr[i] = ld_g(krow + i);
}
// The same for V (vc: position p at + p * HD).
template <int HD, typename KT>
__device__ __forceinline__ void attn_load_v(const KT* vc, int p0, int p1, int lane, AttnBuf<HD, KT>& bf) {
  using Gm = AttnGeom<HD, KT>;
#pragma unroll
  for (int j = 0; j < Gm::NP; ++j) {
    const KT* vrow = vc + (int64_t)min(p0 + j, p1 - 1) * HD + lane * Gm::DPL;
    if constexpr (sizeof(KT) == 2 && Gm::DPL == 1) {
      bf.vr[j][0] = *(gu16_ptr)vrow;
    } else {
#pragma unroll
      for (int w = 0; w < AttnBuf<HD, KT>::VW; ++w) bf.vr[j][w] = ((gu32_ptr)vrow)[w];
    }
  }
}
template <int HD, typename KT>
__device__ __forceinline__ void attn_load(const KT* kc, const KT* vc, int p0, int p1, int lane,
                                          AttnBuf<HD, KT>& bf) {
  attn_load_k<HD, KT>(kc, p0, p1, lane, bf);
  attn_load_v<HD, KT>(vc, p0, p1, lane, bf);
}

// ---------------------------------------------------------------------------
// Matrix-core fragments of v_mfma_f32_16x16x32_bf16.  Lane i supplies row
// (i & 15) of the 16-row A tile and column (i & 15) of the B tile, each with
// the 8 consecutive k of piece (i >> 4) of the 32-wide k-step (both operands
// use the same lane -> k assignment, so products pair matching k).  Result:
// lane i holds D[4 (i >> 4) + j][i & 15], j < 4.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mma16(v4u a, v4u b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Reductions over the 16 lanes of a DPP row (every lane gets the result).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  return fmaxf(v, dpp_f<0x140>(v));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  return v + dpp_f<0x140>(v);
}

// ---- attention on the matrix cores (bf16 cache, head_dim 128) ----------------
// Scores: the query heads of a KV group are the rows of the A operand of
// v_mfma_f32_16x16x32_bf16 (heads past G are zero rows; G <= kMaxGqa = 8
// keeps them in lanes 0-31 of the result) and a block's 16 positions the
// columns of the B operand, so S = Q K^T for the block is 8 instructions: the
// fp32 queries enter as a bf16 pair hi = bf16(q), lo = bf16(q - hi) (16
// significant bits), each multiplied with the exact bf16 keys, fp32
// accumulation.  The k index is permuted so that a lane reads 64 contiguous
// bytes of its position's key row: in k-step ks lane i holds dims
// 32 (i >> 4) + 8 ks .. + 7; the query fragments use the same permutation.
// Result: lane i holds S[head 4 (i >> 4) + j][position i & 15], j < 4.
// The online softmax runs on that layout (row reductions over 16 lanes), so
// a lane keeps m and l of heads 4 (i >> 4) + j.
// Values: O += P V is 8 instructions of v_mfma_f32_16x16x16_bf16 per operand
// half, one per output tile t: A = P (rows = heads, k = the block's positions,
// passed through LDS from the score layout, again as a bf16 hi/lo pair), B =
// the values with the output dims permuted so that a lane's operands come
// from one 16-byte load: column c of tile t is dim 8 c + t, and lane i loads
// dims 8 (i & 15) .. + 7 of positions 4 (i >> 4) .. + 3, one vector each.
// Result: lane i holds O[head 4 (i >> 4) + j][dim 8 (i & 15) + t] in tile t,
// scaled by the same lane's softmax corrections.
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma16k16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

struct AttnQFrag {
  v4u hi[4], lo[4];
};

__device__ __forceinline__ uint32_t bf_pack(uint16_t a, uint16_t b) { return (uint32_t)a | ((uint32_t)b << 16); }

// This lane's query fragments from the rotated queries in LDS (qs[G][128]).
__device__ __forceinline__ void attn_q_frags(const float* qs, int G, int lane, AttnQFrag& f) {
  const int r = lane & 15, d0 = 32 * (lane >> 4);
  const float* qr = qs + min(r, G - 1) * 128 + d0;  // rows past G read a valid row and are zeroed
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const float4 a = *reinterpret_cast<const float4*>(qr + 8 * ks);
    const float4 c = *reinterpret_cast<const float4*>(qr + 8 * ks + 4);
    const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    uint16_t h[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = r < G ? v[e] : 0.f;
      h[e] = f2bf(x);
      lo[e] = f2bf(x - bf1(h[e]));
    }
    f.hi[ks] = v4u{bf_pack(h[0], h[1]), bf_pack(h[2], h[3]), bf_pack(h[4], h[5]), bf_pack(h[6], h[7])};
    f.lo[ks] = v4u{bf_pack(lo[0], lo[1]), bf_pack(lo[2], lo[3]), bf_pack(lo[4], lo[5]), bf_pack(lo[6], lo[7])};
  }
}

// One block of the matrix-core path in registers: kr, dims 32 (lane >> 4) ..
// + 31 of position p0 + (lane & 15)'s key row; vk[i], dims 8 (lane & 15) .. + 7
// of position p0 + 4 (lane >> 4) + i's value row.
struct AttnBufMf {
  v4u kr[4], vk[4];
};

// Issues the block's loads; positions at or past p1 read position p1 - 1
// (their weights are zero).
__device__ __forceinline__ void attn_load_mf(const uint16_t* kc, const uint16_t* vc, int p0, int p1, int lane,
                                             AttnBufMf& bf) {
  const v4u* krow = reinterpret_cast<const v4u*>(kc + (int64_t)min(p0 + (lane & 15), p1 - 1) * 128 + 32 * (lane >> 4));
#pragma unroll
  for (int i = 0; i < 4; ++i) bf.kr[i] = ld_g(krow + i);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    bf.vk[i] = ld_g(reinterpret_cast<const v4u*>(vc + (int64_t)min(p0 + 4 * (lane >> 4) + i, p1 - 1) * 128 +
                                                 8 * (lane & 15)));
}

// Running state: m and l of this lane's heads 4 (lane >> 4) + j, and the
// output tiles (see above).
struct AttnStateMf {
  float m[4], l[4];
  f32x4 o[8];
  __device__ void init() {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m[j] = -INFINITY;
      l[j] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Elements E of two bf16 vectors as one 32-bit word (a's in the low half).
template <int E>
__device__ __forceinline__ uint32_t bf_pair(const v4u& a, const v4u& b) {
  const uint32_t x = a[E >> 1], y = b[E >> 1];
  return E & 1 ? (x >> 16) | (y & 0xFFFF0000u) : (x & 0xFFFFu) | (y << 16);
}

// Online-softmax update with the block [p0, min(p0 + 16, p1)) held in bf.
// pw: this wave's LDS scratch for the weights, [8 heads][16 positions].
__device__ __forceinline__ void attn_compute_mf(const AttnBufMf& bf, const AttnQFrag& qf, int p0, int p1, int G,
                                                int lane, float* pw, AttnStateMf& st) {
  const int np = min(16, p1 - p0), pos = lane & 15, row0 = 4 * (lane >> 4);
  const float scale = 1.0f / sqrtf(128.0f);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    acc = mma16(qf.hi[ks], bf.kr[ks], acc);
    acc = mma16(qf.lo[ks], bf.kr[ks], acc);
  }
  float alpha[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool valid = pos < np && row0 + j < G;
    const float s = valid ? acc[j] * scale : -INFINITY;
    const float mn = fmaxf(st.m[j], row16_max(s));
    alpha[j] = mn == -INFINITY ? 1.f : __expf(st.m[j] - mn);  // 0 on a head's first block; rows past G stay empty
    const float p = valid ? __expf(s - mn) : 0.f;
    st.l[j] = st.l[j] * alpha[j] + row16_sum(p);
    st.m[j] = mn;
    if (row0 + j < G) pw[(row0 + j) * 16 + pos] = p;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) st.o[t][j] *= alpha[j];
  __builtin_amdgcn_wave_barrier();  // the weights are in pw (one wave: its LDS operations stay in order)
  // A operand: weights of head (lane & 15) at positions 4 (lane >> 4) .. + 3
  const int hr = lane & 15;
  const float4 w = *reinterpret_cast<const float4*>(pw + min(hr, G - 1) * 16 + 4 * (lane >> 4));
  const float wv[4] = {w.x, w.y, w.z, w.w};
  uint16_t wh[4], wl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x = hr < G ? wv[i] : 0.f;
    wh[i] = f2bf(x);
    wl[i] = f2bf(x - bf1(wh[i]));
  }
  const s16x4 ah = __builtin_bit_cast(s16x4, u32x2{bf_pack(wh[0], wh[1]), bf_pack(wh[2], wh[3])});
  const s16x4 al = __builtin_bit_cast(s16x4, u32x2{bf_pack(wl[0], wl[1]), bf_pack(wl[2], wl[3])});
  auto tile = [&](auto tc) __attribute__((always_inline)) {
    constexpr int t = decltype(tc)::value;
    const s16x4 b = __builtin_bit_cast(s16x4, u32x2{bf_pair<t>(bf.vk[0], bf.vk[1]), bf_pair<t>(bf.vk[2], bf.vk[3])});
    st.o[t] = mma16k16(ah, b, st.o[t]);
    st.o[t] = mma16k16(al, b, st.o[t]);
  };
  tile(std::integral_constant<int, 0>{});
  tile(std::integral_constant<int, 1>{});
  tile(std::integral_constant<int, 2>{});
  tile(std::integral_constant<int, 3>{});
  tile(std::integral_constant<int, 4>{});
  tile(std::integral_constant<int, 5>{});
  tile(std::integral_constant<int, 6>{});
  tile(std::integral_constant<int, 7>{});
  __builtin_amdgcn_wave_barrier();  // the next block's writes to pw come after these reads
}

// attn_pipeline for the matrix-core path: the wave's blocks b, b + stride, ...
// (below p1), the first already loaded into A.
__device__ __forceinline__ void attn_pipeline_mf(AttnBufMf& A, AttnBufMf& B, const AttnQFrag& qf, const uint16_t* kc,
                                                 const uint16_t* vc, int b, int p1, int stride, int G, int lane,
                                                 float* pw, AttnStateMf& st) {
  for (;;) {
    int n = b + stride;
    if (n >= p1) {
      attn_compute_mf(A, qf, b, p1, G, lane, pw, st);
      return;
    }
    attn_load_mf(kc, vc, n, p1, lane, B);
    attn_compute_mf(A, qf, b, p1, G, lane, pw, st);
    b = n;
    n = b + stride;
    if (n >= p1) {
      attn_compute_mf(B, qf, b, p1, G, lane, pw, st);
      return;
    }
    attn_load_mf(kc, vc, n, p1, lane, A);
    attn_compute_mf(B, qf, b, p1, G, lane, pw, st);
    b = n;
  }
}

// Writes a wave's matrix-core state as G records of (o[128], m, l).
__device__ __forceinline__ void attn_store_state_mf(const AttnStateMf& st, int G, float* out, int lane) {
  const int c = lane & 15, row0 = 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = row0 + j;
    if (h < G) {
      float* oh = out + h * (128 + 2);
#pragma unroll
      for (int t = 0; t < 8; t += 2)  // records are 8-byte aligned (130 floats each)
        *reinterpret_cast<float2*>(oh + 8 * c + t) = make_float2(st.o[t][j], st.o[t + 1][j]);
      if (c == 0) {
        oh[128] = st.m[j];
        oh[129] = st.l[j];
      }
    }
  }
}

// Online-softmax update with the block [p0, min(p0 + NP, p1)) held in bf.
// qs: LDS [G][HD] (rotated queries).  The weight of position j reaches every
// lane by a read of lane j * LPP into a scalar register.
// jr >= 0: row jr of the block takes its values from vcur (this lane's DPL
// dims) instead of bf -- the current position, whose value arrived this step.
template <int HD, typename KT, int GQ = 0>
__device__ __forceinline__ void attn_compute(const AttnBuf<HD, KT>& bf, const float* qs, int p0, int p1, int G,
                                             int lane, AttnState<HD, GQ>& st, int jr = -1,
                                             const float* vcur = nullptr) {
  using Gm = AttnGeom<HD, KT>;
  using Hs = GqaHeads<GQ>;
  constexpr int DPL = Gm::DPL, NP = Gm::NP, LPP = Gm::LPP, EPL = Gm::EPL, GM = Hs::MAX;
  const int np = min(NP, p1 - p0);
  const int my = lane / LPP, part = lane % LPP;  // position and row part this lane scores
  const float scale = 1.0f / sqrtf((float)HD);
  float sc[GM], pv[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) sc[h] = 0.f;
#pragma unroll
  for (int i = 0; i < EPL / 8; ++i) {
#pragma unroll
    for (int h = 0; h < GM; ++h)
      if (Hs::has(h, G)) sc[h] = dot_k<KT>(bf.kr, i, qs + h * HD + part * EPL + i * 8, sc[h]);
  }
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (Hs::has(h, G)) {
      sc[h] += dpp_f<0xB1>(sc[h]);                          // lanes 2j, 2j+1
      if constexpr (LPP >= 4) sc[h] += dpp_f<0x4E>(sc[h]);  // and the other pair of the quad
      if constexpr (LPP == 8) sc[h] += dpp_f<0x141>(sc[h]); // and the other quad of the eight
      const float s = my < np ? sc[h] * scale : -INFINITY;
      const float mn = fmaxf(st.m[h], wave_max(s));
      const float alpha = __expf(st.m[h] - mn);  // 0 on the first block (m = -inf)
      const float p = my < np ? __expf(s - mn) : 0.f;
      st.l[h] = st.l[h] * alpha + wave_sum(p) * (1.0f / LPP);
#pragma unroll
      for (int e = 0; e < DPL; ++e) st.o[h][e] *= alpha;
      st.m[h] = mn;
      pv[h] = p;
    }
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    if (j < np) {
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (Hs::has(h, G)) {
          const float p = rd_lane(pv[h], j * LPP);
          float v[DPL];
          if constexpr (sizeof(KT) == 2) {
            if constexpr (DPL == 2) {
              v[0] = bf_lo(bf.vr[j][0]);
              v[DPL - 1] = bf_hi(bf.vr[j][0]);
            } else {
              v[0] = bf_lo(bf.vr[j][0]);
            }
          } else {
#pragma unroll
            for (int e = 0; e < DPL; ++e) v[e] = __uint_as_float(bf.vr[j][e]);
          }
          if (vcur) {
#pragma unroll
            for (int e = 0; e < DPL; ++e) v[e] = j == jr ? vcur[e] : v[e];
          }
#pragma unroll
          for (int e = 0; e < DPL; ++e) st.o[h][e] = fmaf(p, v[e], st.o[h][e]);
        }
      }
    }
  }
  // Keeps the query reads from LDS inside each block: hoisted out of the
  // block loop they would hold G * EPL values per lane in registers for the
  // whole loop and push the kernel into spills.
  __builtin_amdgcn_wave_barrier();
}

// A wave's blocks b, b + stride, ... (below p1), the first already loaded into
// A: the next block's loads are in flight while the current one is computed.
// Each exit path has its own code, so every path issues a fixed number of
// loads (see gemv_stream).
template <int HD, typename KT, int GQ = 0>
__device__ __forceinline__ void attn_pipeline(AttnBuf<HD, KT>& A, AttnBuf<HD, KT>& B, const float* qs, const KT* kc,
                                              const KT* vc, int b, int p1, int stride, int G, int lane,
                                              AttnState<HD, GQ>& st) {
  for (;;) {
    int n = b + stride;
    if (n >= p1) {
      attn_compute<HD, KT, GQ>(A, qs, b, p1, G, lane, st);
      return;
    }
    attn_load<HD, KT>(kc, vc, n, p1, lane, B);
    attn_compute<HD, KT, GQ>(A, qs, b, p1, G, lane, st);
    b = n;
    n = b + stride;
    if (n >= p1) {
      attn_compute<HD, KT, GQ>(B, qs, b, p1, G, lane, st);
      return;
    }
    attn_load<HD, KT>(kc, vc, n, p1, lane, A);
    attn_compute<HD, KT, GQ>(B, qs, b, p1, G, lane, st);
    b = n;
  }
}

// Writes a wave's state as G records of (o[HD], m, l).
template <int HD, int GQ = 0>
__device__ __forceinline__ void attn_store_state(const AttnState<HD, GQ>& st, int G, float* out, int lane) {
  constexpr int DPL = HD / kWave;
#pragma unroll
  for (int h = 0; h < GqaHeads<GQ>::MAX; ++h) {
    if (GqaHeads<GQ>::has(h, G)) {
      float* oh = out + h * (HD + 2);
#pragma unroll
      for (int e = 0; e < DPL; ++e) oh[lane * DPL + e] = st.o[h][e];
      if (lane == 0) {
        oh[HD] = st.m[h];
        oh[HD + 1] = st.l[h];
      }
    }
  }
}

// Loads the G rotated query heads of a group into LDS (one wave).
template <int HD>
__device__ __forceinline__ void attn_load_q(const float* q, int G, float* qs, int lane) {
  for (int i = lane; i < G * HD; i += kWave) qs[i] = q[i];
  __builtin_amdgcn_wave_barrier();
}

// One wave, positions [p0, p1) in blocks: partial written as G records.
template <int HD, typename KT>
__device__ __forceinline__ void attn_partial(const float* q, const KT* kc, const KT* vc, int p0, int p1, int G,
                                             float* out, float* scratch, int lane) {
  constexpr int NP = AttnGeom<HD, KT>::NP;
  float* qs = scratch;           // [G][HD]
  attn_load_q<HD>(q, G, qs, lane);
  AttnState<HD> st;
  st.init();
  AttnBuf<HD, KT> A, B;
  attn_load<HD, KT>(kc, vc, p0, p1, lane, A);
  attn_pipeline<HD, KT>(A, B, qs, kc, vc, p0, p1, NP, G, lane, st);
  attn_store_state<HD>(st, G, out, lane);
}

// Splits v into bf16 hi = bf16(v) and lo = bf16(v - hi): hi + lo carries 16
// significant bits, the operand pair of the batched matrix-core products.
__device__ __forceinline__ void split_bf16(float v, uint16_t* hi, uint16_t* lo) {
  const uint16_t h = f2bf(v);
  *hi = h;
  *lo = f2bf(v - bf1(h));
}

// Log-sum-exp merge of n partial records laid out [n][G][HD + 2] (stride
// `rec_stride` floats between partials); writes the G normalised outputs to
// out[G][HD] (and, if given, their bf16 hi/lo operand planes).  Records with
// l == 0 (no positions) carry weight 0.  Lane s reads the (m, l) of record s
// (64 records per pass), so the maximum and the weights come from two wave
// reductions; the output loads of all records are then independent of each
// other and stay in flight together.
template <int HD>
__device__ __forceinline__ void attn_merge(const float* part, int n, int G, float* out, int lane, int rec_stride = -1,
                                           uint16_t* out_hi = nullptr, uint16_t* out_lo = nullptr) {
  constexpr int DPL = HD / kWave;
  if (rec_stride < 0) rec_stride = G * (HD + 2);
  for (int h = 0; h < G; ++h) {
    const float* ph = part + h * (HD + 2);
    float M = -INFINITY;
    for (int s0 = 0; s0 < n; s0 += kWave) {
      const int s = min(s0 + lane, n - 1);
      const float ls = ph[(int64_t)s * rec_stride + HD + 1], ms = ph[(int64_t)s * rec_stride + HD];
      if (s0 + lane < n && ls > 0.f) M = fmaxf(M, ms);
    }
    M = wave_max(M);
    float Lsum = 0.f, o[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = 0.f;
    for (int s0 = 0; s0 < n; s0 += kWave) {
      const int s = min(s0 + lane, n - 1);
      const float ls = ph[(int64_t)s * rec_stride + HD + 1], ms = ph[(int64_t)s * rec_stride + HD];
      const float w = s0 + lane < n && ls > 0.f ? __expf(ms - M) : 0.f;  // this lane's record weight
      Lsum += w * (ls > 0.f ? ls : 0.f);
      const int cnt = min(kWave, n - s0);
      for (int j = 0; j < cnt; ++j) {
        const float wj = __shfl(w, j);
        const float* pj = ph + (int64_t)(s0 + j) * rec_stride + lane * DPL;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = fmaf(wj, wj > 0.f ? pj[e] : 0.f, o[e]);
      }
    }
    const float inv = 1.0f / wave_sum(Lsum);
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      out[h * HD + lane * DPL + e] = o[e] * inv;
      if (out_hi) split_bf16(o[e] * inv, out_hi + h * HD + lane * DPL + e, out_lo + h * HD + lane * DPL + e);
    }
  }
}

__device__ __forceinline__ float silu(float u) { return u / (1.0f + __expf(-u)); }

// Loads of data no kernel writes while it runs (the host-built task tables,
// the per-layer weight pointer tables, the per-step argument record) go
// through the constant address space as 32-bit words, so that a load at a
// wave-uniform address uses the scalar cache.  As vector loads -- which the
// 16-bit fields of a task descriptor would otherwise get -- they would queue
// in order behind the weight stream.
typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;
template <class T>
__device__ __forceinline__ T ld_const(const T* p) {
  static_assert(sizeof(T) % 4 == 0, "loaded as 32-bit words");
  struct Words {
    uint32_t w[sizeof(T) / 4];
  } t;
  const_u32_ptr q = (const_u32_ptr)p;
#pragma unroll
  for (int k = 0; k < (int)(sizeof(T) / 4); ++k) t.w[k] = q[k];
  return __builtin_bit_cast(T, t);
}
__device__ __forceinline__ Task load_task(const Task* tasks, int i) { return ld_const(tasks + i); }

// ---------------------------------------------------------------------------
// Cache addressing and token lookup shared by the single-sequence and batched paths.
__device__ __forceinline__ int64_t kv_off(const Params& P, int l, int b, int g, int p) {
  return ((((int64_t)l * P.B + b) * P.nkv + g) * P.max_seq + p) * P.hd;
}

// Stores one K or V element in the cache's element type.
__device__ __forceinline__ void kv_store(const Params& P, void* cache, int64_t off, float v) {
  if (P.kv_f32) static_cast<float*>(cache)[off] = v;
  else static_cast<uint16_t*>(cache)[off] = f2bf(v);
}

// Token id of batch row b, clamped into [0, V) so that a bad id can never
// address outside the embedding table; a clamp latches ST_BADTOKEN.
__device__ __forceinline__ int token_of(const Params& P, const Step& S, int b) {
  const int t = S.tokens[(int64_t)b * S.tok_stride];
  if (t >= 0 && t < P.V) return t;
  atomicCAS(&P.status[1], ST_OK, ST_BADTOKEN);
  return 0;
}


// ---------------------------------------------------------------------------
// GEMV task helpers shared by the per-operator kernels and the megakernel.

template <int R>
__device__ __forceinline__ float pick(const float (&y)[R], int i) {
  float v = y[0];
#pragma unroll
  for (int r = 1; r < R; ++r) v = i == r ? y[r] : v;
  return v;
}

// GEMV-type task (QKV, O, GU, DOWN, LM) with its operator fixed at compile
// time: where its rows are ...
// Rows of task d in the matrices W0 (QKV: the task's own matrix; GU: gate)
// and W1 (GU: up).
template <int TT>
__device__ __forceinline__ void gemv_setup_w(const Params& P, const Task& d, const uint16_t* W0, const uint16_t* W1,
                                             GemvRows<TaskShape<TT>::R>& g) {
  constexpr int R = TaskShape<TT>::R;
  int K = P.H;
  if constexpr (TT == TT_O) K = P.nq * P.hd;
  else if constexpr (TT == TT_DOWN) K = P.F;
  g.nvec = K / 8;
  g.stride = K / 8;
  g.split = R;
  if constexpr (TT == TT_QKV) {
    const uint16_t* W = W0;
    g.base0 = reinterpret_cast<const v4u*>(W + (int64_t)d.a1 * K);
    if (d.a3) {  // one RoPE pair: rows a1 and a1 + hd/2
      g.base1 = reinterpret_cast<const v4u*>(W + (int64_t)(d.a1 + d.a3) * K);
      g.split = 1;
      g.mask = 3;
    } else {
      g.base1 = g.base0;
      g.mask = (1u << d.a2) - 1;
    }
  } else if constexpr (TT == TT_GU) {  // rows: gate a1.., then up a1..
    g.base0 = reinterpret_cast<const v4u*>(W0 + (int64_t)d.a1 * K);
    g.base1 = reinterpret_cast<const v4u*>(W1 + (int64_t)d.a1 * K);
    g.split = R / 2;
    const uint32_t half = (1u << d.a2) - 1;
    g.mask = half | (half << (R / 2));
  } else {
    g.base0 = reinterpret_cast<const v4u*>(W0 + (int64_t)d.a1 * K);
    g.base1 = g.base0;
    g.mask = (1u << d.a2) - 1;
  }
}

template <int TT>
__device__ __forceinline__ void gemv_put(float* res, int* ids, int j, int task, const float (&y)[TaskShape<TT>::R],
                                         int lane) {
  constexpr int R = TaskShape<TT>::R;
  if (lane < R) res[j * R + lane] = pick<R>(y, lane);
  if (lane == 0) ids[j] = task;
}

// The task of pool slot p of this workgroup, or `count` past its end.  The
// dispatcher deals workgroups to the XCDs in turn (workgroup b runs on XCD
// b % kXcds).  When the grid is a multiple of kXcds, the workgroups of one
// XCD share one contiguous kXcds-th of the task list, dealt to them in runs of
// kWaves tasks; otherwise the runs go to all workgroups in turn.  (Dealing
// runs to all workgroups in turn makes XCD x read the same few consecutive
// rows out of every kXcds runs -- for 8 KB rows a fixed 32 KB slice of every
// 256 KB -- and the XCDs then finish up to a fifth apart.)
__device__ __forceinline__ int slot_task(uint32_t p, int count) {
  const int n = gridDim.x, run = (int)(p / kWaves), k = (int)(p % kWaves);
  if (n % kXcds) {
    const int t = (run * n + (int)blockIdx.x) * kWaves + k;
    return t < count ? t : count;
  }
  const int per = (count + kXcds - 1) / kXcds, x = (int)blockIdx.x % kXcds, j = (int)blockIdx.x / kXcds;
  const int t = (run * (n / kXcds) + j) * kWaves + k;
  return t < per && x * per + t < count ? x * per + t : count;
}

// The next pool slot's task of this wave, or `count` when the pool is empty
// or the wave's result slots are full (j results kept, one task in hand).
__device__ __forceinline__ int gemv_next(uint32_t* pool, int j, int count, int lane) {
  if (j + 2 > kMaxTasksPerWave) return count;
  uint32_t p = 0;
  if (lane == 0) p = lds_add(pool, 1u);
  p = __builtin_amdgcn_readfirstlane(p);
  return slot_task(p, count);
}

}  // namespace mk
