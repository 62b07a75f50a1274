// Batched decode (B > 1 sequences per step).
//
// With B sequences every weight byte streamed from HBM serves B dot products,
// so the projections become skinny GEMMs Y[B, N] = A[B, K] . W[N, K]^T: at 8
// sequences that is 8 FMAs per weight element and at 64 it is 64, beyond what
// the vector ALUs sustain at HBM speed.  The products therefore run on the
// matrix cores (v_mfma_f32_16x16x32_bf16: bf16 operands, fp32 accumulation),
// the matrix-matrix form that the summary of the Hazy Research throughput
// megakernel (hakusoku, "全てのGPUを購入したので、徹底的にそのGPUを活用します。",
// section 高スループットMegakernelの設計と工夫 / 命令セットの再設計) gives for
// throughput-oriented batches, as against matrix-vector bodies for latency.
// The activation operand is written, when it is produced, as two bf16 planes
// hi = bf16(v) and lo = bf16(v - hi) -- by mk_b_norm for the normalised
// inputs, the merge kernel for the attention output, the gate/up epilogue for
// the SwiGLU output -- and every fragment goes through the matrix core twice
// (W.hi + W.lo).  hi + lo holds 16 significant bits, so the products see the
// activations at close to fp32 precision (relative error <= 2^-17) instead of
// bf16's 2^-9; the matrix cores have the throughput to spare at these batch
// sizes.  Everything else (residual stream, RoPE, softmax, norms) is fp32.
//
// Work split: a workgroup of four waves owns four groups of two 16-row weight
// tiles (one group per wave) and one range of K.  The activation operand is
// shared by every row, so the workgroup stages it through LDS in 128- or
// 256-column chunks (double-buffered, one barrier per chunk) and each wave
// reads its fragments there; re-reading them from L2 per wave made the
// activation traffic several times the weight traffic and bounded these
// kernels by L2 bandwidth.  Each wave streams its own weight rows with a
// chunk of k-steps in flight.  Operators with few row groups also split K
// across workgroups: partial sums go to a buffer and a finishing launch adds
// them in a fixed order and runs the epilogue.
//
// Operator order per layer: norm -> QKV(+RoPE, KV append) -> split-KV
// attention -> merge -> O(+residual) -> norm -> gate/up(+SwiGLU) ->
// down(+residual); then the final norm, the LM head with per-tile argmax
// partials, and the argmax.
#include "device.h"
#include "kernels.h"

namespace mk {

// The matrix-core fragments (mma16, in device.h): the weight tile is the A
// operand (rows = weight rows), the activation tile the B operand (columns =
// batch rows); the result holds D[weight row][batch row].

// Rows of one wave's group of two 16-row weight tiles, per operator.
//   QKV (RT 2): groups [0, nq*hd/32) are query, then key, then value groups.
//     A query/key group pairs tile rows i0.. and i0 + hd/2.. of one head
//     (i0 < hd/2, a multiple of 16), so the RoPE pair (i, i + hd/2) of every
//     row lands in the same thread; a value group is 32 consecutive rows.
//   O, DOWN, LM (RT 2): 32 consecutive rows.
//   GU (RT 2): the same 16 rows of W_gate and of W_up.
constexpr int kRT = 2;  // 16-row tiles per wave

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
      G.W[0] = G.W[1] = isq ? ld_const(P.wq + l) : ld_const(P.wk + l);
      G.N = (isq ? P.nq : P.nkv) * hd;
      G.row0[0] = head * hd + i0;
      G.row0[1] = head * hd + hd / 2 + i0;
    } else {
      G.mat = 2;
      G.W[0] = G.W[1] = ld_const(P.wv + l);
      G.N = P.nkv * hd;
      G.row0[0] = (g - nqg - nkg) * 32;
      G.row0[1] = G.row0[0] + 16;
    }
  } else if constexpr (TT == TT_O) {
    G.K = P.nq * hd;
    G.N = P.H;
    G.W[0] = G.W[1] = ld_const(P.wo + l);
    G.row0[0] = g * 32;
    G.row0[1] = g * 32 + 16;
  } else if constexpr (TT == TT_GU) {
    G.K = P.H;
    G.N = P.F;
    G.W[0] = ld_const(P.w_gate + l);
    G.W[1] = ld_const(P.w_up + l);
    G.row0[0] = G.row0[1] = g * 16;
  } else if constexpr (TT == TT_DOWN) {
    G.K = P.F;
    G.N = P.H;
    G.W[0] = G.W[1] = ld_const(P.w_down + l);
    G.row0[0] = g * 32;
    G.row0[1] = g * 32 + 16;
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
    const int64_t tok = l == 0 ? (int64_t)token_of(P, S, b) * H : 0;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int row = G.row0[r] + m;
      if (row < G.N) {
        const float xin = l == 0 ? bf1(P.embed[tok + row]) : P.xs[((int64_t)l * P.B + b) * H + row];
        P.xmid[((int64_t)l * P.B + b) * H + row] = xin + y[r];
      }
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
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int row = G.row0[r] + m;
      if (row < G.N) P.xs[((int64_t)(l + 1) * P.B + b) * H + row] = P.xmid[((int64_t)l * P.B + b) * H + row] + y[r];
    }
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

// ---- the staged-activation GEMM core ------------------------------------------
// An activation chunk in LDS: [2 planes][Bp rows][KC + 8] bf16; the 16-byte
// row pad keeps the 16 rows of one fragment read on distinct banks.
template <int BT, int KC>
struct Chunk {
  static constexpr int Bp = 16 * BT;
  static constexpr int STEPS = KC / 32;              // k-steps per chunk (= weight steps in flight)
  static constexpr int ROW = KC + 8;                 // padded row, elements
  static constexpr int ELEMS = 2 * Bp * ROW;         // one buffer
  static constexpr int PIECES = 2 * Bp * (KC / 8);   // 16-byte pieces per chunk
  static constexpr int PER_THREAD = PIECES / (kBgemmWaves * kWave);
};
template <int BT, int KC>
constexpr int chunk_lds_bytes() { return 2 * Chunk<BT, KC>::ELEMS * 2; }

// This thread's pieces of chunk c (columns [c*KC, c*KC + KC)) of the operand
// planes A [2][Bp][K]; columns at or past K read a clamped address and are
// zeroed, so every load is issued unconditionally.
template <int BT, int KC>
__device__ __forceinline__ void chunk_load(const uint16_t* A, int K, int c, v4u (&cr)[Chunk<BT, KC>::PER_THREAD]) {
  using C = Chunk<BT, KC>;
#pragma unroll
  for (int i = 0; i < C::PER_THREAD; ++i) {
    const int idx = threadIdx.x + i * kBgemmWaves * kWave;
    const int piece = idx % (KC / 8), row = (idx / (KC / 8)) % C::Bp, plane = idx / (C::Bp * (KC / 8));
    const int k = c * KC + piece * 8;
    const v4u v = ld_g(reinterpret_cast<const v4u*>(A + ((int64_t)plane * C::Bp + row) * K + min(k, K - 8)));
    cr[i] = k < K ? v : v4u{0u, 0u, 0u, 0u};
  }
}

template <int BT, int KC>
__device__ __forceinline__ void chunk_store(uint16_t* buf, const v4u (&cr)[Chunk<BT, KC>::PER_THREAD]) {
  using C = Chunk<BT, KC>;
#pragma unroll
  for (int i = 0; i < C::PER_THREAD; ++i) {
    const int idx = threadIdx.x + i * kBgemmWaves * kWave;
    const int piece = idx % (KC / 8), row = (idx / (KC / 8)) % C::Bp, plane = idx / (C::Bp * (KC / 8));
    *reinterpret_cast<v4u*>(buf + (plane * C::Bp + row) * C::ROW + piece * 8) = cr[i];
  }
}

// The weight fragments of k-step s (global step index) of the wave's two
// tiles.  Row-major weights: this lane's 16 bytes of its row (16 rows x 64
// bytes per wave load).  Tiled weights (16 x 32 blocks stored as the
// fragments of one wave load): this lane's 16 bytes of the tile's block s,
// so one wave load reads 1 KB in one piece.
template <int RT, bool TILED>
__device__ __forceinline__ void weights_load(v4u (&wb)[RT], const v4u* const (&wr)[RT], int s, int nvec, int piece) {
  if constexpr (TILED) {
    const int b = min(s, nvec / 4 - 1);  // past K: any in-bounds block (the activations are zero there)
#pragma unroll
    for (int r = 0; r < RT; ++r) wb[r] = ld_w(wr[r] + 64 * b);
  } else {
    const int v = min(4 * s + piece, nvec - 1);  // past K: any in-bounds vector (the activations are zero there)
#pragma unroll
    for (int r = 0; r < RT; ++r) wb[r] = ld_w(wr[r] + v);
  }
}

// acc[r][t] += W_r . (A_t.hi + A_t.lo)^T for k-step `ks` of the chunk in buf.
template <int RT, int BT, int KC>
__device__ __forceinline__ void chunk_mma(const v4u (&wb)[RT], const uint16_t* buf, int ks, int lane,
                                          f32x4 (&acc)[RT][BT]) {
  using C = Chunk<BT, KC>;
  const int col = ks * 32 + (lane >> 4) * 8;
#pragma unroll
  for (int t = 0; t < BT; ++t) {
    const int row = t * 16 + (lane & 15);
    const v4u h = *reinterpret_cast<const v4u*>(buf + row * C::ROW + col);
    const v4u lo = *reinterpret_cast<const v4u*>(buf + (C::Bp + row) * C::ROW + col);
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[r][t] = mma16(wb[r], h, acc[r][t]);
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[r][t] = mma16(wb[r], lo, acc[r][t]);
  }
}

// One workgroup: the K chunks [c0, c1) of the four tile groups of its waves.
// Chunk ci+1 (activations and weights) is in flight while chunk ci is
// multiplied; the last chunk is peeled so that every loop iteration issues
// the same loads.  Returns the accumulators of this wave's two tiles.
template <int RT, int BT, int KC, bool TILED>
__device__ __forceinline__ void staged_gemm(const uint16_t* A, int K, const v4u* const (&wr)[RT], int c0, int c1,
                                            uint16_t* lds, int lane, f32x4 (&acc)[RT][BT]) {
  using C = Chunk<BT, KC>;
  constexpr int ST = C::STEPS;
  const int piece = lane >> 4, nvec = K / 8;
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < BT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  v4u cr[C::PER_THREAD];
  v4u wb[ST][RT];
  chunk_load<BT, KC>(A, K, c0, cr);
#pragma unroll
  for (int d = 0; d < ST; ++d) weights_load<RT, TILED>(wb[d], wr, c0 * ST + d, nvec, piece);
  chunk_store<BT, KC>(lds, cr);
  __syncthreads();
  int ci = c0;
  for (; ci + 1 < c1; ++ci) {
    const uint16_t* buf = lds + ((ci - c0) & 1) * C::ELEMS;
    chunk_load<BT, KC>(A, K, ci + 1, cr);
#pragma unroll
    for (int d = 0; d < ST; ++d) {
      chunk_mma<RT, BT, KC>(wb[d], buf, d, lane, acc);
      weights_load<RT, TILED>(wb[d], wr, (ci + 1) * ST + d, nvec, piece);
    }
    chunk_store<BT, KC>(lds + ((ci + 1 - c0) & 1) * C::ELEMS, cr);
    __syncthreads();
  }
  const uint16_t* buf = lds + ((ci - c0) & 1) * C::ELEMS;
#pragma unroll
  for (int d = 0; d < ST; ++d) chunk_mma<RT, BT, KC>(wb[d], buf, d, lane, acc);
}

// Row groups per operator (each is one wave's two tiles).
template <int TT>
__device__ __forceinline__ int group_count(const Params& P) {
  if constexpr (TT == TT_QKV) return (P.nq + 2 * P.nkv) * P.hd / 32;
  else if constexpr (TT == TT_GU) return (P.F + 15) / 16;
  else if constexpr (TT == TT_LM) return (P.V + 31) / 32;
  else return (P.H + 31) / 32;  // O, DOWN
}

// This lane's weight stream of each tile: its row (row-major weights) or its
// 16 bytes in the tile's first block (tiled weights: N % 16 == 0, K % 32 == 0).
template <int TT, bool TILED>
__device__ __forceinline__ void group_pointers(const Params& P, int l, int g, int lane, GroupRows& G,
                                               const v4u* (&wr)[kRT]) {
  G = group_rows<TT>(P, l, g);
#pragma unroll
  for (int r = 0; r < kRT; ++r) {
    if constexpr (TILED) {
      const int row0 = min(G.row0[r], G.N - 16);  // a tile past the end re-reads the last one (discarded)
      wr[r] = reinterpret_cast<const v4u*>(G.W[r] + (int64_t)row0 * G.K) + lane;
    } else {
      const int row = min(G.row0[r] + (lane & 15), G.N - 1);  // rows past the end repeat the last (discarded)
      wr[r] = reinterpret_cast<const v4u*>(G.W[r] + (int64_t)row * G.K);
    }
  }
}

// Split-K partial layout: part[((kz * ngroups + g) * RT + r) * 16 + m][b].
__device__ __forceinline__ int64_t part_index(int kz, int ngroups, int g, int r, int m, int b, int Bp) {
  return ((((int64_t)kz * ngroups + g) * kRT + r) * 16 + m) * Bp + b;
}

// The projection kernel: grid (ceil(groups / (4 * GPW)), splits of K); wave w
// of workgroup x owns the GPW row groups (x * 4 + w) * GPW + i.  With 64
// batch rows and many groups two groups per wave pay: every activation
// fragment read from LDS then feeds four tiles instead of two (one group per
// wave reads four bytes of LDS per weight byte, near the LDS bandwidth).
// With one split the epilogue runs here, straight from each wave's
// accumulators; otherwise the partial sums go to P.bpart for the finishing
// launch.
template <int TT, int BT, int KC, bool TILED, int GPW>
__device__ __forceinline__ void bgemm(const Params& P, const Step& S, int l) {
  constexpr int RT = kRT * GPW;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);
  unsigned long long* best = reinterpret_cast<unsigned long long*>(smem + chunk_lds_bytes<BT, KC>());  // [64]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ngroups = group_count<TT>(P);
  const int g0 = (blockIdx.x * kBgemmWaves + wave) * GPW;
  if constexpr (TT == TT_LM) {
    if (threadIdx.x < kMaxBatch) best[threadIdx.x] = 0;
  }
  GroupRows G[GPW];
  const v4u* wr[RT];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const v4u* w2[kRT];
    group_pointers<TT, TILED>(P, l, min(g0 + gi, ngroups - 1), lane, G[gi], w2);  // spares repeat the last group
#pragma unroll
    for (int r = 0; r < kRT; ++r) wr[gi * kRT + r] = w2[r];
  }
  const int nch = (G[0].K + KC - 1) / KC, ks = gridDim.y, per = (nch + ks - 1) / ks;
  const int c0 = blockIdx.y * per, c1 = min(c0 + per, nch);
  f32x4 acc[RT][BT];
  staged_gemm<RT, BT, KC, TILED>(operand_of<TT>(P), G[0].K, wr, c0, c1, lds, lane, acc);
  if (ks == 1) {
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      if (g0 + gi < ngroups) {
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int m = 4 * (lane >> 4) + j, b = t * 16 + (lane & 15);
            float y[kRT];
#pragma unroll
            for (int r = 0; r < kRT; ++r) y[r] = acc[gi * kRT + r][t][j];
            if (b < P.B) bgemm_epilogue<TT, kRT>(P, S, l, G[gi], m, b, y, best);
          }
      }
    }
    if constexpr (TT == TT_LM) {
      __syncthreads();
      if (threadIdx.x < P.B && best[threadIdx.x])
        __hip_atomic_fetch_max(&P.lm_part[threadIdx.x], best[threadIdx.x], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      if (g0 + gi >= ngroups) continue;
#pragma unroll
      for (int r = 0; r < kRT; ++r)
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            P.bpart[part_index(blockIdx.y, ngroups, g0 + gi, r, 4 * (lane >> 4) + j, t * 16 + (lane & 15), 16 * BT)] =
                acc[gi * kRT + r][t][j];
    }
  }
}

// Finishing launch of a split projection: one workgroup per row group, one
// thread per (row, batch column) of its 16-row tiles (16 * Bp threads).  The
// splits' partial sums are read in their stored order (batch columns
// contiguous, so the loads coalesce), four splits' loads at a time, and added
// in split order (fixed, so results do not depend on timing).  The sums then
// pass through LDS so that the epilogue runs with consecutive threads on
// consecutive rows of one batch row, which keeps its stores and residual loads
// contiguous; with threads along the batch every store went to another row
// (8 sequences of 4K tokens at the 8B shape: 31 us of finishing launches per
// layer, 70B shape at 64 sequences: 101 us).
template <int TT>
__device__ __forceinline__ void bgemm_finish(const Params& P, const Step& S, int l, int ks) {
  __shared__ unsigned long long best[kMaxBatch];
  __shared__ float sy[kRT][16][kMaxBatch + 1];  // padded: the row-wise reads hit distinct banks
  const int g = blockIdx.x, ngroups = group_count<TT>(P), Bp = P.Bp, n = 16 * Bp, e = threadIdx.x;
  const GroupRows G = group_rows<TT>(P, l, g);
  const int64_t kstride = (int64_t)ngroups * kRT * n;  // between splits (part_index layout)
  const float* part = P.bpart + (int64_t)g * kRT * n + e;
  float y[kRT];
#pragma unroll
  for (int r = 0; r < kRT; ++r) y[r] = 0.f;
#pragma unroll 4
  for (int kz = 0; kz < ks; ++kz)
#pragma unroll
    for (int r = 0; r < kRT; ++r) y[r] += part[kz * kstride + r * n];
#pragma unroll
  for (int r = 0; r < kRT; ++r) sy[r][e / Bp][e % Bp] = y[r];  // element (m, b) = (e / Bp, e % Bp)
  __syncthreads();
  const int m = e & 15, b = e >> 4;
  if (b < P.B) {
    float v[kRT];
#pragma unroll
    for (int r = 0; r < kRT; ++r) v[r] = sy[r][m][b];
    bgemm_epilogue<TT, kRT>(P, S, l, G, m, b, v, best);
  }
}

// Chunk width by batch tiles: 256 columns at 16 rows, 128 at 32 and 64 (LDS).
template <int BT> struct BChunk { static constexpr int KC = BT == 1 ? 256 : 128; };

#define MK_BGEMM(name, TT, BT, SUF, TILED, GPW)                                                               \
  extern "C" __global__ __launch_bounds__(kBgemmWaves * kWave) void name##_b##BT##SUF(Params P,               \
                                                                                       const Step* Sd,         \
                                                                                       int layer) {            \
    const Step S = ld_const(Sd);                                                                              \
    bgemm<TT, BT, BChunk<BT>::KC, TILED, GPW>(P, S, layer);                                                   \
  }
#define MK_BGEMM_ALL(name, TT)                                                                                \
  MK_BGEMM(name, TT, 1, , false, 1) MK_BGEMM(name, TT, 2, , false, 1) MK_BGEMM(name, TT, 4, , false, 1)       \
  MK_BGEMM(name, TT, 1, _t, true, 1) MK_BGEMM(name, TT, 2, _t, true, 1) MK_BGEMM(name, TT, 4, _t, true, 1)    \
  MK_BGEMM(name, TT, 4, _g2, false, 2) MK_BGEMM(name, TT, 4, _t_g2, true, 2)
MK_BGEMM_ALL(mk_b_qkv, TT_QKV)
MK_BGEMM_ALL(mk_b_o, TT_O)
MK_BGEMM_ALL(mk_b_gu, TT_GU)
MK_BGEMM_ALL(mk_b_down, TT_DOWN)
MK_BGEMM_ALL(mk_b_lm, TT_LM)

#define MK_BFIN(name, TT)                                                                                     \
  extern "C" __global__ __launch_bounds__(16 * kMaxBatch) void name(Params P, const Step* Sd, int layer, int ks) { \
    const Step S = ld_const(Sd);                                                                              \
    bgemm_finish<TT>(P, S, layer, ks);                                                                        \
  }
MK_BFIN(mk_b_fin_qkv, TT_QKV)
MK_BFIN(mk_b_fin_o, TT_O)
MK_BFIN(mk_b_fin_gu, TT_GU)
MK_BFIN(mk_b_fin_down, TT_DOWN)

// RMSNorm of one batch row into the bf16 operand planes of ax:
// ax[b] = x * (mean(x^2) + eps)^-1/2 * gamma as hi/lo.  kind 0: attention norm
// of `layer` (x = embedding row at layer 0), 1: FFN norm, 2: final norm.  One
// workgroup per row; each thread keeps up to kNormGroups groups of 8 values
// in registers between the two passes; the sum of squares is reduced in a
// fixed order.
constexpr int kNormGroups = 4;  // rows up to 8192 in registers (longer rows are re-read)
extern "C" __global__ __launch_bounds__(kNormThreads) void mk_b_norm(Params P, const Step* Sd, int layer, int kind) {
  __shared__ float part[kNormThreads / kWave];
  const Step S = ld_const(Sd);
  const int b = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t H = P.H;
  const float* xf = nullptr;
  const uint16_t* xb = nullptr;
  const uint16_t* gamma;
  if (kind == 0) {
    gamma = ld_const(P.attn_norm + layer);
    if (layer == 0) xb = P.embed + (int64_t)token_of(P, S, b) * H;
    else xf = P.xs + ((int64_t)layer * P.B + b) * H;
  } else if (kind == 1) {
    gamma = ld_const(P.ffn_norm + layer);
    xf = P.xmid + ((int64_t)layer * P.B + b) * H;
  } else {
    gamma = P.final_norm;
    xf = P.xs + ((int64_t)P.L * P.B + b) * H;
  }
  auto load8 = [&](int i, float (&v)[8]) __attribute__((always_inline)) {
    if (xf) {
      const float4 a = *reinterpret_cast<const float4*>(xf + i), c = *reinterpret_cast<const float4*>(xf + i + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
    } else {
      const v4u u = ld_g(reinterpret_cast<const v4u*>(xb + i));
      v[0] = bf_lo(u.x); v[1] = bf_hi(u.x); v[2] = bf_lo(u.y); v[3] = bf_hi(u.y);
      v[4] = bf_lo(u.z); v[5] = bf_hi(u.z); v[6] = bf_lo(u.w); v[7] = bf_hi(u.w);
    }
  };
  constexpr int NT = kNormThreads * 8;  // elements per pass over the row
  float v[kNormGroups][8];
  float ss = 0.f;
#pragma unroll
  for (int g = 0; g < kNormGroups; ++g) {
    const int i = g * NT + threadIdx.x * 8;
    if (i < P.H) {
      load8(i, v[g]);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf(v[g][j], v[g][j], ss);
    }
  }
  for (int i = kNormGroups * NT + threadIdx.x * 8; i < P.H; i += NT) {
    float w[8];
    load8(i, w);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(w[j], w[j], ss);
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
  auto emit = [&](int i, const float (&w)[8]) __attribute__((always_inline)) {
    const v4u g = ld_g(reinterpret_cast<const v4u*>(gamma + i));
    const float gm[8] = {bf_lo(g.x), bf_hi(g.x), bf_lo(g.y), bf_hi(g.y), bf_lo(g.z), bf_hi(g.z), bf_lo(g.w), bf_hi(g.w)};
    uint16_t h[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) split_bf16(w[j] * inv * gm[j], &h[j], &l[j]);
    v4u ph, pl;
    ph.x = h[0] | (uint32_t)h[1] << 16; ph.y = h[2] | (uint32_t)h[3] << 16;
    ph.z = h[4] | (uint32_t)h[5] << 16; ph.w = h[6] | (uint32_t)h[7] << 16;
    pl.x = l[0] | (uint32_t)l[1] << 16; pl.y = l[2] | (uint32_t)l[3] << 16;
    pl.z = l[4] | (uint32_t)l[5] << 16; pl.w = l[6] | (uint32_t)l[7] << 16;
    *reinterpret_cast<v4u*>(hi + i) = ph;
    *reinterpret_cast<v4u*>(lo + i) = pl;
  };
#pragma unroll
  for (int g = 0; g < kNormGroups; ++g) {
    const int i = g * NT + threadIdx.x * 8;
    if (i < P.H) emit(i, v[g]);
  }
  for (int i = kNormGroups * NT + threadIdx.x * 8; i < P.H; i += NT) {
    float w[8];
    load8(i, w);
    emit(i, w);
  }
}

// Next tokens from the LM head's argmax keys; clears the keys for the next step.
extern "C" __global__ void mk_b_argmax(Params P, const Step* Sd) {
  const Step S = ld_const(Sd);
  const int b = threadIdx.x;
  if (b >= P.B) return;
  const unsigned long long k = P.lm_part[b];
  S.out[b] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
  if (!(fabsf(argmax_key_value(k)) <= 3.0e38f)) atomicCAS(&P.status[1], ST_OK, ST_NONFINITE);
  P.lm_part[b] = 0ull;
}

// Test entry: Y[b][n] = sum_k W[n][k] (A.hi[b][k] + A.lo[b][k]) for bf16 W
// [N, K] (row-major, or tiled) and A [2][Bp][K] (rows B..Bp-1 zero): the same
// staged core, each wave owning 32 consecutive rows, one split.
template <int BT, bool TILED>
__device__ __forceinline__ void t_bgemm(const uint16_t* W, const uint16_t* A, float* Y, int N, int K, int B) {
  constexpr int KC = BChunk<BT>::KC;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * kBgemmWaves + wave) * 32;
  const v4u* wr[kRT];
#pragma unroll
  for (int r = 0; r < kRT; ++r) {
    if constexpr (TILED)
      wr[r] = reinterpret_cast<const v4u*>(W + (int64_t)min(row0 + r * 16, N - 16) * K) + lane;
    else
      wr[r] = reinterpret_cast<const v4u*>(W + (int64_t)min(row0 + r * 16 + (lane & 15), N - 1) * K);
  }
  f32x4 acc[kRT][BT];
  staged_gemm<kRT, BT, KC, TILED>(A, K, wr, 0, (K + KC - 1) / KC, lds, lane, acc);
#pragma unroll
  for (int r = 0; r < kRT; ++r)
#pragma unroll
    for (int t = 0; t < BT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = t * 16 + (lane & 15), row = row0 + r * 16 + 4 * (lane >> 4) + j;
        if (b < B && row < N) Y[(int64_t)b * N + row] = acc[r][t][j];
      }
}
extern "C" __global__ __launch_bounds__(kBgemmWaves * kWave) void mk_t_bgemm_kernel(const uint16_t* W,
                                                                                     const uint16_t* A, float* Y,
                                                                                     int N, int K, int B, int tiled) {
  const int bt = (B + 15) / 16;
  if (tiled) {
    if (bt == 1) t_bgemm<1, true>(W, A, Y, N, K, B);
    else if (bt == 2) t_bgemm<2, true>(W, A, Y, N, K, B);
    else t_bgemm<4, true>(W, A, Y, N, K, B);
  } else {
    if (bt == 1) t_bgemm<1, false>(W, A, Y, N, K, B);
    else if (bt == 2) t_bgemm<2, false>(W, A, Y, N, K, B);
    else t_bgemm<4, false>(W, A, Y, N, K, B);
  }
}

// Row-major W [N][K] bf16 -> the tiled layout read by the batched projections:
// block (i, j) of 16 rows x 32 columns at element offset (i * K/32 + j) * 512,
// holding lane l's 8 elements W[16i + l % 16][32j + 8 (l / 16) .. + 8] at
// offset 8 l (the fragment lane l supplies to one matrix-core k-step).  One
// thread per 16-byte vector of the destination.
extern "C" __global__ __launch_bounds__(256) void mk_tile_kernel(const uint16_t* src, uint16_t* dst, int64_t N,
                                                                 int64_t K) {
  const int64_t nv = N * K / 8, bpr = K / 32;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nv; v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t blk = v / 64, i = blk / bpr, j = blk % bpr;
    const int l = (int)(v % 64);
    const int64_t row = 16 * i + (l & 15), col = 32 * j + 8 * (l >> 4);
    *reinterpret_cast<v4u*>(dst + 8 * v) = ld_g(reinterpret_cast<const v4u*>(src + row * K + col));
  }
}

// LDS bytes of the batched projection kernels and the test entry, by batch
// tiles (the argmax keys of the LM head come on top).
int b_lds_bytes(int bt) {
  return bt == 1 ? chunk_lds_bytes<1, BChunk<1>::KC>() : bt == 2 ? chunk_lds_bytes<2, BChunk<2>::KC>()
                                                                 : chunk_lds_bytes<4, BChunk<4>::KC>();
}

}  // namespace mk
