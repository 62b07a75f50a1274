// Batched decode (B > 1 sequences per step).
//
// With B sequences every weight byte streamed from HBM serves B dot products,
// so the projections become skinny GEMMs Y[B, N] = A[B, K] . W[N, K]^T: at 8
// sequences that is 8 FMAs per weight element and at 64 it is 64, beyond what
// the vector ALUs sustain at HBM speed.  The products therefore run on the
// matrix cores (v_mfma_f32_16x16x32_bf16: bf16 operands, fp32 accumulation),
// the skinny-GEMM form the Hazy Research megakernel write-up ("Look Ma, No
// Bubbles!", its batched throughput section) gives for serving-size batches.
// The activation operand is written, when it is produced, as two bf16 planes
// hi = bf16(v) and lo = bf16(v - hi) -- by mk_b_norm for the normalised
// inputs, the merge kernel for the attention output, the gate/up epilogue for
// the SwiGLU output -- and every fragment goes through the matrix core twice
// (W.hi + W.lo).  hi + lo holds 16 significant bits, so the products see the
// activations at close to fp32 precision (relative error <= 2^-17) instead of
// bf16's 2^-9; the matrix cores have the throughput to spare at these batch
// sizes.  Everything else (residual stream, RoPE, softmax, norms) is fp32.
//
// Operator order per layer (one launch each): norm -> QKV(+RoPE, KV append) ->
// split-KV attention -> merge -> O(+residual) -> norm -> gate/up(+SwiGLU) ->
// down(+residual); then the final norm, the LM head with per-tile argmax
// partials, and the argmax.
#include "device.h"
#include "kernels.h"

namespace mk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Operand fragments of v_mfma_f32_16x16x32_bf16.  Lane i supplies row (i & 15)
// of its 16-row tile and the 8 consecutive k of piece (i >> 4) of the 32-wide
// k-step; the weight tile (A) and the activation tile (B) use the same lane ->
// k assignment, so products pair matching k.  Result: lane i holds
// D[4 (i >> 4) + j][i & 15], j < 4 (weight row, batch row).
__device__ __forceinline__ f32x4 mma16(v4u w, v4u a, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), __builtin_bit_cast(bf16x8, a), c, 0,
                                                 0, 0);
}

// One wave: acc[r][t] += W_r . (A_t.hi + A_t.lo)^T over the k-steps [s0, s1)
// (32 columns each).  wr[r] / ar[t]: this lane's weight row / operand row (hi
// plane; the lo plane is lo_off vectors further) as 16-byte vectors; nvec =
// K / 8.  D k-steps of every operand stay in flight: rounds of D steps, each
// slot refilled right after it is consumed, the last round only consuming.
// No load is predicated (see gemv_run): with EXACT every step is in range;
// otherwise addresses are clamped and the operand of an out-of-range step
// is zeroed.
template <int RT, int BT, int D, bool EXACT>
__device__ __forceinline__ void mma_load(v4u (&wb)[RT], v4u (&ah)[BT], v4u (&al)[BT], const v4u* const (&wr)[RT],
                                         const v4u* const (&ar)[BT], int64_t lo_off, int nvec, int s, int piece) {
  const int v = EXACT ? 4 * s + piece : min(4 * s + piece, nvec - 1);
#pragma unroll
  for (int r = 0; r < RT; ++r) wb[r] = ld_w(wr[r] + v);
#pragma unroll
  for (int t = 0; t < BT; ++t) {
    ah[t] = ld_g(ar[t] + v);
    al[t] = ld_g(ar[t] + lo_off + v);
  }
}

template <int RT, int BT, bool EXACT>
__device__ __forceinline__ void mma_consume(const v4u (&wb)[RT], const v4u (&ah)[BT], const v4u (&al)[BT], bool ok,
                                            f32x4 (&acc)[RT][BT]) {
  const v4u z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int t = 0; t < BT; ++t) {
    const v4u h = EXACT || ok ? ah[t] : z, l = EXACT || ok ? al[t] : z;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      acc[r][t] = mma16(wb[r], h, acc[r][t]);
      acc[r][t] = mma16(wb[r], l, acc[r][t]);
    }
  }
}

template <int RT, int BT, int D, bool EXACT>
__device__ __forceinline__ void mma_run(const v4u* const (&wr)[RT], const v4u* const (&ar)[BT], int64_t lo_off,
                                        int nvec, int s0, int s1, int lane, f32x4 (&acc)[RT][BT]) {
  const int piece = lane >> 4;
  const int nrounds = (s1 - s0 + D - 1) / D;
  if (nrounds <= 0) return;
  v4u wb[D][RT], ah[D][BT], al[D][BT];
#pragma unroll
  for (int d = 0; d < D; ++d) mma_load<RT, BT, D, EXACT>(wb[d], ah[d], al[d], wr, ar, lo_off, nvec, s0 + d, piece);
  for (int rd = 0; rd + 1 < nrounds; ++rd) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int s = s0 + rd * D + d;
      mma_consume<RT, BT, EXACT>(wb[d], ah[d], al[d], s < s1 && 4 * s + piece < nvec, acc);
      mma_load<RT, BT, D, EXACT>(wb[d], ah[d], al[d], wr, ar, lo_off, nvec, s + D, piece);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int s = s0 + (nrounds - 1) * D + d;
    mma_consume<RT, BT, EXACT>(wb[d], ah[d], al[d], s < s1 && 4 * s + piece < nvec, acc);
  }
}

// Splits the K steps of a tile over the NW waves and runs the wave's share;
// the exact variant when every wave gets the same multiple of D steps.
template <int RT, int BT, int NW, int D>
__device__ __forceinline__ void mma_wave(const v4u* const (&wr)[RT], const v4u* const (&ar)[BT], int64_t lo_off,
                                         int nvec, int wave, int lane, f32x4 (&acc)[RT][BT]) {
  const int nsteps = (nvec + 3) / 4, per = (nsteps + NW - 1) / NW;
  const int s0 = min(wave * per, nsteps), s1 = min(s0 + per, nsteps);
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < BT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nvec % 4 == 0 && nsteps % NW == 0 && per % D == 0) mma_run<RT, BT, D, true>(wr, ar, lo_off, nvec, s0, s1, lane, acc);
  else mma_run<RT, BT, D, false>(wr, ar, lo_off, nvec, s0, s1, lane, acc);
}

// Row layout of one workgroup's group of RT 16-row tiles, per operator.
//   QKV (RT 2): groups [0, nq*hd/32) are query, then key, then value groups.
//     A query/key group pairs tile rows i0.. and i0 + hd/2.. of one head
//     (i0 < hd/2, a multiple of 16), so the RoPE pair (i, i + hd/2) of every
//     row lands in the same thread; a value group is 32 consecutive rows.
//   O, DOWN (RT 1): 16 consecutive rows.
//   GU (RT 2): the same 16 rows of W_gate and of W_up.
//   LM (RT 2): 32 consecutive rows.
struct GroupRows {
  const uint16_t* W[2];  // matrix of each tile
  int row0[2];           // first row of each tile
  int N, K;              // matrix rows (for clamping) and columns
  int mat;               // QKV: 0 q, 1 k, 2 v
};

template <int TT>
__device__ __forceinline__ GroupRows group_rows(const Params& P, int l, int g) {
  GroupRows G{};
  const int hd = P.hd;
  if constexpr (TT == TT_QKV) {
    G.K = P.H;
    const int per_head = hd / 32, nqg = P.nq * per_head, nkg = P.nkv * per_head;
    if (g < nqg + nkg) {
      const bool isq = g < nqg;
      const int gg = isq ? g : g - nqg, head = gg / per_head, i0 = (gg % per_head) * 16;
      G.mat = isq ? 0 : 1;
      G.W[0] = G.W[1] = isq ? P.wq[l] : P.wk[l];
      G.N = (isq ? P.nq : P.nkv) * hd;
      G.row0[0] = head * hd + i0;
      G.row0[1] = head * hd + hd / 2 + i0;
    } else {
      G.mat = 2;
      G.W[0] = G.W[1] = P.wv[l];
      G.N = P.nkv * hd;
      G.row0[0] = (g - nqg - nkg) * 32;
      G.row0[1] = G.row0[0] + 16;
    }
  } else if constexpr (TT == TT_O) {
    G.K = P.nq * hd;
    G.N = P.H;
    G.W[0] = G.W[1] = P.wo[l];
    G.row0[0] = G.row0[1] = g * 16;
  } else if constexpr (TT == TT_GU) {
    G.K = P.H;
    G.N = P.F;
    G.W[0] = P.w_gate[l];
    G.W[1] = P.w_up[l];
    G.row0[0] = G.row0[1] = g * 16;
  } else if constexpr (TT == TT_DOWN) {
    G.K = P.F;
    G.N = P.H;
    G.W[0] = G.W[1] = P.w_down[l];
    G.row0[0] = G.row0[1] = g * 16;
  } else {
    G.K = P.H;
    G.N = P.V;
    G.W[0] = G.W[1] = P.tied ? P.embed : P.lm_head;
    G.row0[0] = g * 32;
    G.row0[1] = g * 32 + 16;
  }
  return G;
}

template <int TT>
__device__ __forceinline__ const uint16_t* operand_of(const Params& P) {
  if constexpr (TT == TT_O) return P.ao;
  else if constexpr (TT == TT_DOWN) return P.ah;
  else return P.ax;
}

// Epilogue of one output element pair: m = row within the tiles, b = batch row,
// y[r] = the finished dot product of tile r.
template <int TT, int RT>
__device__ __forceinline__ void bgemm_epilogue(const Params& P, const Step& S, int l, const GroupRows& G, int m, int b,
                                               const float (&y)[RT], unsigned long long* best) {
  const int64_t H = P.H;
  if constexpr (TT == TT_QKV) {
    const int r0 = G.row0[0] + m, r1 = G.row0[1] + m;
    if (G.mat == 2) {
      kv_store(P, P.vcache, kv_off(P, l, b, r0 / P.hd, S.pos) + r0 % P.hd, y[0]);
      kv_store(P, P.vcache, kv_off(P, l, b, r1 / P.hd, S.pos) + r1 % P.hd, y[1]);
    } else {  // rotate the pair (r0, r1 = r0 + hd/2) by the position's angles
      const int half = P.hd / 2, i = r0 % P.hd;
      const float c = P.rope_cos[(int64_t)S.pos * half + i], sn = P.rope_sin[(int64_t)S.pos * half + i];
      const float lo = y[0] * c - y[1] * sn, hi = y[1] * c + y[0] * sn;
      if (G.mat == 0) {
        float* q = P.q + ((int64_t)l * P.B + b) * P.nq * P.hd;
        q[r0] = lo;
        q[r1] = hi;
      } else {
        const int64_t o = kv_off(P, l, b, r0 / P.hd, S.pos);
        kv_store(P, P.kcache, o + i, lo);
        kv_store(P, P.kcache, o + i + half, hi);
      }
    }
  } else if constexpr (TT == TT_O) {
    const int row = G.row0[0] + m;
    if (row < G.N) {
      const float xin = l == 0 ? bf1(P.embed[(int64_t)token_of(P, S, b) * H + row])
                               : P.xs[((int64_t)l * P.B + b) * H + row];
      P.xmid[((int64_t)l * P.B + b) * H + row] = xin + y[0];
    }
  } else if constexpr (TT == TT_GU) {
    const int row = G.row0[0] + m;
    if (row < G.N) {
      const float hv = silu(y[0]) * y[1];
      P.h[((int64_t)l * P.B + b) * P.F + row] = hv;
      uint16_t* hi = P.ah + (int64_t)b * P.F + row;
      split_bf16(hv, hi, hi + (int64_t)P.Bp * P.F);
    }
  } else if constexpr (TT == TT_DOWN) {
    const int row = G.row0[0] + m;
    if (row < G.N) P.xs[((int64_t)(l + 1) * P.B + b) * H + row] = P.xmid[((int64_t)l * P.B + b) * H + row] + y[0];
  } else {
    unsigned long long k = 0;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int row = G.row0[r] + m;
      if (row < G.N) {
        if (S.logits) S.logits[(int64_t)b * P.V + row] = y[r];
        const unsigned long long c = argmax_key(y[r], (uint32_t)row);
        k = c > k ? c : k;
      }
    }
    if (k) __hip_atomic_fetch_max(&best[b], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// One workgroup = one group of RT row tiles x all batch tiles.  Its NW waves
// split the K columns; each wave's partial accumulators go to LDS and are
// summed in wave order (a fixed order: the result does not depend on timing).
template <int TT, int RT, int BT, int NW, int D>
__device__ __forceinline__ void bgemm(const Params& P, const Step& S, int l) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* red = reinterpret_cast<float*>(smem);                                    // [NW][RT][BT][4][64]
  unsigned long long* best = reinterpret_cast<unsigned long long*>(red + NW * RT * BT * 256);  // [64]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const GroupRows G = group_rows<TT>(P, l, blockIdx.x);
  if constexpr (TT == TT_LM) {
    if (threadIdx.x < kMaxBatch) best[threadIdx.x] = 0;
  }
  const int nvec = G.K / 8;
  const v4u* wr[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int row = min(G.row0[r] + (lane & 15), G.N - 1);  // rows past the end repeat the last (discarded)
    wr[r] = reinterpret_cast<const v4u*>(G.W[r] + (int64_t)row * G.K);
  }
  const uint16_t* A = operand_of<TT>(P);
  const v4u* ar[BT];
#pragma unroll
  for (int t = 0; t < BT; ++t) ar[t] = reinterpret_cast<const v4u*>(A + (int64_t)(t * 16 + (lane & 15)) * G.K);
  f32x4 acc[RT][BT];
  mma_wave<RT, BT, NW, D>(wr, ar, (int64_t)P.Bp * nvec, nvec, wave, lane, acc);
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < BT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[(((wave * RT + r) * BT + t) * 4 + j) * 64 + lane] = acc[r][t][j];
  __syncthreads();
  for (int e = threadIdx.x; e < BT * 256; e += NW * kWave) {
    const int t = e >> 8, j = (e >> 6) & 3, ln = e & 63;
    const int b = t * 16 + (ln & 15), m = 4 * (ln >> 4) + j;
    if (b >= P.B) continue;
    float y[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      float s = 0.f;
      for (int w = 0; w < NW; ++w) s += red[(((w * RT + r) * BT + t) * 4 + j) * 64 + ln];
      y[r] = s;
    }
    bgemm_epilogue<TT, RT>(P, S, l, G, m, b, y, best);
  }
  if constexpr (TT == TT_LM) {
    __syncthreads();
    if (threadIdx.x < P.B && best[threadIdx.x])
      __hip_atomic_fetch_max(&P.lm_part[threadIdx.x], best[threadIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Prefetch depth by batch tiles: the operand fragments share the in-flight
// register budget with the weight fragments.
template <int BT> struct BDepth { static constexpr int D = BT == 1 ? 8 : 4; };

#define MK_BGEMM(name, TT, RT, BT)                                                                            \
  extern "C" __global__ __launch_bounds__(kBgemmWaves * kWave) void name##_b##BT(Params P, const Step* Sd,     \
                                                                                  int layer) {                \
    const Step S = *Sd;                                                                                       \
    bgemm<TT, RT, BT, kBgemmWaves, BDepth<BT>::D>(P, S, layer);                                                \
  }
#define MK_BGEMM_ALL(name, TT, RT) MK_BGEMM(name, TT, RT, 1) MK_BGEMM(name, TT, RT, 2) MK_BGEMM(name, TT, RT, 4)
MK_BGEMM_ALL(mk_b_qkv, TT_QKV, 2)
MK_BGEMM_ALL(mk_b_o, TT_O, 1)
MK_BGEMM_ALL(mk_b_gu, TT_GU, 2)
MK_BGEMM_ALL(mk_b_down, TT_DOWN, 1)
MK_BGEMM_ALL(mk_b_lm, TT_LM, 2)

// RMSNorm of one batch row into the bf16 operand buffer ax:
// ax[b] = bf16(x * (mean(x^2) + eps)^-1/2 * gamma).  kind 0: attention norm of
// `layer` (x = embedding row at layer 0), 1: FFN norm, 2: final norm.  One
// workgroup per row; the sum of squares is reduced in a fixed order.
extern "C" __global__ __launch_bounds__(kNormThreads) void mk_b_norm(Params P, const Step* Sd, int layer, int kind) {
  __shared__ float part[kNormThreads / kWave];
  const Step S = *Sd;
  const int b = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t H = P.H;
  const float* xf = nullptr;
  const uint16_t* xb = nullptr;
  const uint16_t* gamma;
  if (kind == 0) {
    gamma = P.attn_norm[layer];
    if (layer == 0) xb = P.embed + (int64_t)token_of(P, S, b) * H;
    else xf = P.xs + ((int64_t)layer * P.B + b) * H;
  } else if (kind == 1) {
    gamma = P.ffn_norm[layer];
    xf = P.xmid + ((int64_t)layer * P.B + b) * H;
  } else {
    gamma = P.final_norm;
    xf = P.xs + ((int64_t)P.L * P.B + b) * H;
  }
  float ss = 0.f;
  for (int i = threadIdx.x; i < P.H; i += kNormThreads) {
    const float v = xf ? xf[i] : bf1(xb[i]);
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / kWave; ++w) tot += part[w];
  const float inv = 1.0f / sqrtf(tot / (float)P.H + P.eps);
  uint16_t* hi = P.ax + (int64_t)b * H;
  uint16_t* lo = hi + (int64_t)P.Bp * H;
  for (int i = threadIdx.x; i < P.H; i += kNormThreads) {
    const float v = xf ? xf[i] : bf1(xb[i]);
    split_bf16(v * inv * bf1(gamma[i]), hi + i, lo + i);
  }
}

// Next tokens from the LM head's argmax keys; clears the keys for the next step.
extern "C" __global__ void mk_b_argmax(Params P, const Step* Sd) {
  const Step S = *Sd;
  const int b = threadIdx.x;
  if (b >= P.B) return;
  const unsigned long long k = P.lm_part[b];
  S.out[b] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
  if (!(fabsf(argmax_key_value(k)) <= 3.0e38f)) atomicCAS(&P.status[1], ST_OK, ST_NONFINITE);
  P.lm_part[b] = 0ull;
}

// Test entry: Y[b][n] = sum_k W[n][k] (A.hi[b][k] + A.lo[b][k]) for bf16 W
// [N, K] and A [2][Bp][K] (rows B..Bp-1 zero), one 16-row tile per
// workgroup, through the same wave loop and workgroup reduction as the
// operators.
template <int BT>
__device__ __forceinline__ void t_bgemm(const uint16_t* W, const uint16_t* A, float* Y, int N, int K, int B) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* red = reinterpret_cast<float*>(smem);
  constexpr int NW = kBgemmWaves, D = BDepth<BT>::D;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int row0 = blockIdx.x * 16, nvec = K / 8;
  const v4u* wr[1] = {reinterpret_cast<const v4u*>(W + (int64_t)min(row0 + (lane & 15), N - 1) * K)};
  const v4u* ar[BT];
#pragma unroll
  for (int t = 0; t < BT; ++t) ar[t] = reinterpret_cast<const v4u*>(A + (int64_t)(t * 16 + (lane & 15)) * K);
  f32x4 acc[1][BT];
  mma_wave<1, BT, NW, D>(wr, ar, (int64_t)16 * BT * nvec, nvec, wave, lane, acc);
#pragma unroll
  for (int t = 0; t < BT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[((wave * BT + t) * 4 + j) * 64 + lane] = acc[0][t][j];
  __syncthreads();
  for (int e = threadIdx.x; e < BT * 256; e += NW * kWave) {
    const int t = e >> 8, j = (e >> 6) & 3, ln = e & 63;
    const int b = t * 16 + (ln & 15), row = row0 + 4 * (ln >> 4) + j;
    if (b >= B || row >= N) continue;
    float s = 0.f;
    for (int w = 0; w < NW; ++w) s += red[((w * BT + t) * 4 + j) * 64 + ln];
    Y[(int64_t)b * N + row] = s;
  }
}
extern "C" __global__ __launch_bounds__(kBgemmWaves * kWave) void mk_t_bgemm_kernel(const uint16_t* W,
                                                                                     const uint16_t* A, float* Y,
                                                                                     int N, int K, int B) {
  const int bt = (B + 15) / 16;
  if (bt == 1) t_bgemm<1>(W, A, Y, N, K, B);
  else if (bt == 2) t_bgemm<2>(W, A, Y, N, K, B);
  else t_bgemm<4>(W, A, Y, N, K, B);
}

}  // namespace mk
