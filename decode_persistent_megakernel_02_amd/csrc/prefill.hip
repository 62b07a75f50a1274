// Batched prefill: every prompt position of every sequence in one pass per
// chunk of rows, instead of one decode step per position.  The projections run
// as matrix-core GEMMs (the host calls rocBLAS on bf16 operands); this file
// holds the work between them: the embedding gather, RMSNorm with the operand
// split, RoPE with the KV append, causal attention, SwiGLU and the argmax.
// What each step computes is the decode step's operator, for all positions at
// once ("Compilar LLM en un MegaKernel para lograr inferencia de baja
// latencia", "Parte 1. Compilador": the model's operators); prefill as the
// throughput counterpart of decode ("Cómo la fusión de kernels CUDA acelera la
// inferencia de LLM", section "Comprueba si la fusión ha ayudado"), on
// matrix-by-matrix instructions (the hakusoku summary page, section
// 命令セットの再設計).
#include "device.h"
#include "prefill.h"

namespace mk {
namespace {

constexpr int kT = 256;  // threads per workgroup of every kernel here

// Sum over the workgroup (all threads call it); red holds kT / 64 floats.
__device__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();  // red may still be read from the previous call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kT / 64; ++i) t += red[i];
  return t;
}

__device__ __forceinline__ void split_store(uint16_t* hi, uint16_t* lo, int64_t i, float v) {
  const uint16_t h = f2bf(v);
  hi[i] = h;
  lo[i] = f2bf(v - bf1(h));
}

__global__ __launch_bounds__(kT) void k_embed(Params P, const int32_t* tokens, int tok_stride, int c, int p0,
                                              float* X) {
  const int r = blockIdx.x, b = r / c, i = r % c;
  int t = tokens[(int64_t)b * tok_stride + p0 + i];
  if (t < 0 || t >= P.V) {
    if (threadIdx.x == 0) atomicCAS(&P.status[1], ST_OK, ST_BADTOKEN);
    t = 0;
  }
  const uint16_t* e = P.embed + (int64_t)t * P.H;
  float* x = X + (int64_t)r * P.H;
  for (int k = threadIdx.x; k < P.H; k += kT) x[k] = bf1(e[k]);
}

__global__ __launch_bounds__(kT) void k_add_norm_split(Params P, float* X, const float* T, int ldt,
                                                       const uint16_t* gamma, int rstride, int roff, uint16_t* hi,
                                                       uint16_t* lo) {
  __shared__ float red[kT / 64];
  const int o = blockIdx.x, src = o * rstride + roff, H = P.H;
  float* x = X + (int64_t)src * H;
  float ss = 0.f;
  for (int k = threadIdx.x; k < H; k += kT) {
    float v = x[k];
    if (T) {
      v += T[(int64_t)src * ldt + k];
      x[k] = v;
    }
    ss = fmaf(v, v, ss);
  }
  const float inv = 1.0f / sqrtf(block_sum(ss, red) / (float)H + P.eps);
  for (int k = threadIdx.x; k < H; k += kT) split_store(hi, lo, (int64_t)o * H + k, x[k] * inv * bf1(gamma[k]));
}

__global__ __launch_bounds__(kT) void k_rope_kv(Params P, int l, float* QKV, int ldq, int c, int p0) {
  const int r = blockIdx.x, b = r / c, p = p0 + r % c;
  const int half = P.hd / 2, qd = P.nq * P.hd, kd = P.nkv * P.hd;
  float* row = QKV + (int64_t)r * ldq;
  for (int t = threadIdx.x; t < (P.nq + P.nkv) * half; t += kT) {
    const int hh = t / half, i = t % half;
    float* base = row + (hh < P.nq ? hh * P.hd : qd + (hh - P.nq) * P.hd);
    const float cs = P.rope_cos[(int64_t)p * half + i], sn = P.rope_sin[(int64_t)p * half + i];
    const float y0 = base[i], y1 = base[i + half];
    const float a = y0 * cs - y1 * sn, z = y1 * cs + y0 * sn;
    base[i] = a;
    base[i + half] = z;
    if (hh >= P.nq) {
      const int64_t off = kv_off(P, l, b, hh - P.nq, p);
      kv_store(P, P.kcache, off + i, a);
      kv_store(P, P.kcache, off + i + half, z);
    }
  }
  for (int t = threadIdx.x; t < kd; t += kT)
    kv_store(P, P.vcache, kv_off(P, l, b, t / P.hd, p) + t % P.hd, row[qd + kd + t]);
}

// Causal attention.  Workgroup (query block, KV head g, sequence b) holds 64
// query rows: Qb = 64 / G positions times the G query heads of g (row
// q = position index * G + head index).  Keys and values stream through LDS
// in blocks of 64 positions; each block's scores (4 x 4 per thread), an online
// softmax (4 threads per row) and the output update (8 rows x HD/32 dims per
// thread) follow one another between barriers.
template <typename KT>
__device__ __forceinline__ float kv_ld(const KT* p) {
  if constexpr (std::is_same<KT, float>::value) return *p;
  else return bf1(*p);
}

template <int HD, typename KT>
__global__ __launch_bounds__(kT) void k_attention(Params P, int l, const float* QKV, int ldq, int c, int p0,
                                                  uint16_t* hi, uint16_t* lo) {
  extern __shared__ float sm[];
  constexpr int KP = HD + 1, DPT = HD / 32;
  float* Qs = sm;             // [64][HD], scaled by 1/sqrt(HD)
  float* Ks = Qs + 64 * HD;   // [64][KP]
  float* Vs = Ks + 64 * KP;   // [64][HD]
  float* Ps = Vs + 64 * HD;   // [64][65] scores, then weights
  float* mrow = Ps + 64 * 65; // running maximum per row
  float* lrow = mrow + 64;    // running sum per row
  float* arow = lrow + 64;    // this block's rescale factor per row
  const int G = P.nq / P.nkv, Qb = 64 / G;
  const int i0 = blockIdx.x * Qb, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int npos = min(Qb, c - i0);  // valid query positions of this block
  const float scale = 1.0f / sqrtf((float)HD);
  for (int e = t; e < 64 * HD; e += kT) {
    const int q = e / HD, d = e % HD, qi = q / G, gi = q % G;
    Qs[e] = qi < npos ? QKV[(int64_t)(b * c + i0 + qi) * ldq + (g * G + gi) * HD + d] * scale : 0.f;
  }
  if (t < 64) {
    mrow[t] = -INFINITY;
    lrow[t] = 0.f;
  }
  const int pmax = p0 + i0 + npos - 1;  // last key position any row of the block needs
  const KT* kc = static_cast<const KT*>(P.kcache) + kv_off(P, l, b, g, 0);
  const KT* vc = static_cast<const KT*>(P.vcache) + kv_off(P, l, b, g, 0);
  float o[8][DPT];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int d = 0; d < DPT; ++d) o[a][d] = 0.f;
  const int rg = t / 16, kg = t % 16;  // scores: rows 4 rg .. 4 rg + 3, keys 4 kg .. 4 kg + 3
  const int og = t / 32, dg = t % 32;  // output: rows 8 og .. 8 og + 7, dims DPT dg ..
  for (int j0 = 0; j0 <= pmax; j0 += 64) {
    __syncthreads();  // the previous block's keys, values and weights are consumed
    for (int e = t; e < 64 * HD; e += kT) {
      const int j = e / HD, d = e % HD;
      const bool in = j0 + j <= pmax;
      Ks[j * KP + d] = in ? kv_ld(kc + (int64_t)(j0 + j) * HD + d) : 0.f;
      Vs[j * HD + d] = in ? kv_ld(vc + (int64_t)(j0 + j) * HD + d) : 0.f;
    }
    __syncthreads();
    float s[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int k = 0; k < 4; ++k) s[a][k] = 0.f;
    for (int d = 0; d < HD; ++d) {
      float qv[4], kv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) qv[a] = Qs[(4 * rg + a) * HD + d];
#pragma unroll
      for (int k = 0; k < 4; ++k) kv[k] = Ks[(4 * kg + k) * KP + d];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int k = 0; k < 4; ++k) s[a][k] = fmaf(qv[a], kv[k], s[a][k]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int q = 4 * rg + a, pos = p0 + i0 + q / G;  // the row's query position
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = j0 + 4 * kg + k;
        Ps[q * 65 + 4 * kg + k] = j <= pos ? s[a][k] : -INFINITY;
      }
    }
    __syncthreads();
    {  // online softmax: 4 threads per row, 16 keys each
      const int q = t / 4, part = t % 4;
      float mx = -INFINITY;
      for (int k = 0; k < 16; ++k) mx = fmaxf(mx, Ps[q * 65 + part * 16 + k]);
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      mx = fmaxf(mx, __shfl_xor(mx, 2));
      const float mold = mrow[q], mnew = fmaxf(mold, mx);
      float sum = 0.f;
      for (int k = 0; k < 16; ++k) {
        const float sv = Ps[q * 65 + part * 16 + k];
        const float w = sv == -INFINITY ? 0.f : __expf(sv - mnew);
        Ps[q * 65 + part * 16 + k] = w;
        sum += w;
      }
      sum += __shfl_xor(sum, 1);
      sum += __shfl_xor(sum, 2);
      // every row has at least key 0 in the first block, so mnew is finite
      const float alpha = mold == -INFINITY ? 0.f : __expf(mold - mnew);
      __syncthreads();  // every thread of the row has read mrow before it changes
      if (part == 0) {
        mrow[q] = mnew;
        lrow[q] = lrow[q] * alpha + sum;
        arow[q] = alpha;
      }
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const float al = arow[8 * og + a];
#pragma unroll
      for (int d = 0; d < DPT; ++d) o[a][d] *= al;
    }
    for (int k = 0; k < 64; ++k) {
      float vv[DPT];
#pragma unroll
      for (int d = 0; d < DPT; ++d) vv[d] = Vs[k * HD + dg * DPT + d];
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const float w = Ps[(8 * og + a) * 65 + k];
#pragma unroll
        for (int d = 0; d < DPT; ++d) o[a][d] = fmaf(w, vv[d], o[a][d]);
      }
    }
  }
  __syncthreads();
  const int qd = P.nq * HD;
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int q = 8 * og + a, qi = q / G, gi = q % G;
    if (qi >= npos) continue;
    const float inv = 1.0f / lrow[q];
    const int64_t base = (int64_t)(b * c + i0 + qi) * qd + (g * G + gi) * HD + dg * DPT;
#pragma unroll
    for (int d = 0; d < DPT; ++d) split_store(hi, lo, base + d, o[a][d] * inv);
  }
}

// Causal attention on the matrix cores (bf16 cache, head_dim 128), the same
// rows as k_attention: four waves, each 16 of the block's 64 query rows (wave
// w: rows 16 w .. 16 w + 15), keys in blocks of 64 positions.
// Scores: S = Q K^T as v_mfma_f32_16x16x32_bf16 per 16-key tile, the fp32
// queries (scaled by 1/sqrt(128)) as a bf16 pair hi + lo, each times the exact
// bf16 keys, fp32 accumulation.  Lane i supplies query row i & 15 and key
// i & 15 of the tile, both with dims 32 ks + 8 (i >> 4) .. + 7 in k-step ks,
// so a key fragment is 16 contiguous bytes of its cache row.  Result: lane i
// holds S[row 4 (i >> 4) + j][key i & 15], j < 4; the online softmax works on
// that layout (row reductions over 16 lanes), so a lane keeps the running
// maximum and sum of rows 4 (i >> 4) + j.
// Values: O += P V as v_mfma_f32_16x16x16_bf16 per 16-key step and 16-dim
// output tile tt, P passed through LDS into the A layout (lane i: row i & 15,
// keys 4 (i >> 4) .. + 3) as a bf16 pair, the values with dims permuted so
// that column c of tile tt is dim 8 c + tt: lane i loads dims 8 (i & 15) .. + 7
// of keys 4 (i >> 4) .. + 3, one 16-byte vector each, and takes element tt of
// each for tile tt.  Result: lane i holds O[row 4 (i >> 4) + j][dim 8 (i & 15)
// + tt], rescaled with the same lane's softmax corrections.
__device__ __forceinline__ uint32_t pack_bf2(uint16_t a, uint16_t b) { return (uint32_t)a | ((uint32_t)b << 16); }
// bf16 element e (0..7) of a 16-byte vector
__device__ __forceinline__ short bf_elem(const v4u& v, int e) {
  const uint32_t w = v[e >> 1];
  return (short)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
}

__global__ __launch_bounds__(kT) void k_attention_mma(Params P, int l, const float* QKV, int ldq, int c, int p0,
                                                      uint16_t* hi, uint16_t* lo) {
  constexpr int HD = 128, PB = 68;
  __shared__ float pbuf[4 * 16 * PB];
  const int G = P.nq / P.nkv, Qb = 64 / G;
  const int i0 = blockIdx.x * Qb, g = blockIdx.y, b = blockIdx.z;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int npos = min(Qb, c - i0), pmax = p0 + i0 + npos - 1;
  const float scale = 1.0f / sqrtf((float)HD);
  v4u qh[4], ql[4];
  {
    const int q = 16 * w + lr, qi = q / G, gi = q % G;
    const bool valid = qi < npos;
    const float* src = QKV + (int64_t)(b * c + i0 + (valid ? qi : 0)) * ldq + (g * G + gi) * HD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint16_t h8[8], l8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = valid ? src[32 * ks + 8 * lq + e] * scale : 0.f;
        h8[e] = f2bf(x);
        l8[e] = f2bf(x - bf1(h8[e]));
      }
      qh[ks] = v4u{pack_bf2(h8[0], h8[1]), pack_bf2(h8[2], h8[3]), pack_bf2(h8[4], h8[5]), pack_bf2(h8[6], h8[7])};
      ql[ks] = v4u{pack_bf2(l8[0], l8[1]), pack_bf2(l8[2], l8[3]), pack_bf2(l8[4], l8[5]), pack_bf2(l8[6], l8[7])};
    }
  }
  int qpos[4];  // query position of the lane's result rows
#pragma unroll
  for (int j = 0; j < 4; ++j) qpos[j] = p0 + i0 + (16 * w + 4 * lq + j) / G;
  const uint16_t* kc = static_cast<const uint16_t*>(P.kcache) + kv_off(P, l, b, g, 0);
  const uint16_t* vc = static_cast<const uint16_t*>(P.vcache) + kv_off(P, l, b, g, 0);
  float* pb = pbuf + w * 16 * PB;
  float m[4], lsum[4];
  f32x4 o[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m[j] = -INFINITY;
    lsum[j] = 0.f;
  }
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) o[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const v4u zero{0u, 0u, 0u, 0u};
  for (int j0 = 0; j0 <= pmax; j0 += 64) {
    f32x4 s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int key = j0 + 16 * t + lr;
      const bool kin = key <= pmax;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const v4u kf = kin ? *reinterpret_cast<const v4u*>(kc + (int64_t)key * HD + 32 * ks + 8 * lq) : zero;
        s[t] = mma16(qh[ks], kf, s[t]);
        s[t] = mma16(ql[ks], kf, s[t]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float v = j0 + 16 * t + lr <= qpos[j] ? s[t][j] : -INFINITY;
        s[t][j] = v;
        mx = fmaxf(mx, v);
      }
      mx = row16_max(mx);
      const float mnew = fmaxf(m[j], mx);
      const float alpha = m[j] == -INFINITY ? 0.f : __expf(m[j] - mnew);
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float pv = s[t][j] == -INFINITY ? 0.f : __expf(s[t][j] - mnew);
        s[t][j] = pv;
        sum += pv;
      }
      lsum[j] = lsum[j] * alpha + row16_sum(sum);
      m[j] = mnew;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) o[tt][j] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) pb[(4 * lq + j) * PB + 16 * t + lr] = s[t][j];
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint16_t ph[4], pl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = pb[lr * PB + 16 * t + 4 * lq + e];
        ph[e] = f2bf(x);
        pl[e] = f2bf(x - bf1(ph[e]));
      }
      const s16x4 pa_h{(short)ph[0], (short)ph[1], (short)ph[2], (short)ph[3]};
      const s16x4 pa_l{(short)pl[0], (short)pl[1], (short)pl[2], (short)pl[3]};
      v4u vv[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = j0 + 16 * t + 4 * lq + kk;
        vv[kk] = key <= pmax ? *reinterpret_cast<const v4u*>(vc + (int64_t)key * HD + 8 * lr) : zero;
      }
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const s16x4 bv{bf_elem(vv[0], tt), bf_elem(vv[1], tt), bf_elem(vv[2], tt), bf_elem(vv[3], tt)};
        o[tt] = mma16k16(pa_h, bv, o[tt]);
        o[tt] = mma16k16(pa_l, bv, o[tt]);
      }
    }
    __syncthreads();  // the weights are read before the next block writes them
  }
  const int qd = P.nq * HD;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = 16 * w + 4 * lq + j, qi = q / G, gi = q % G;
    if (qi >= npos) continue;
    const float inv = 1.0f / lsum[j];
    const int64_t base = (int64_t)(b * c + i0 + qi) * qd + (g * G + gi) * HD + 8 * lr;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) split_store(hi, lo, base + tt, o[tt][j] * inv);
  }
}

constexpr int attn_lds_bytes(int hd) { return 4 * (64 * hd + 64 * (hd + 1) + 64 * hd + 64 * 65 + 3 * 64); }

__global__ __launch_bounds__(kT) void k_swiglu_split(Params P, const float* GU, uint16_t* hi, uint16_t* lo) {
  const int r = blockIdx.x, F = P.F;
  const float* g = GU + (int64_t)r * 2 * F;
  for (int k = threadIdx.x; k < F; k += kT) split_store(hi, lo, (int64_t)r * F + k, silu(g[k]) * g[F + k]);
}

__global__ __launch_bounds__(kT) void k_fold(const float* src, int lds, int off, float* dst, int ldd, int n) {
  const int r = blockIdx.x;
  const float* a = src + (int64_t)r * lds;
  float* d = dst + (int64_t)r * ldd;
  if (off) {
    const float* b = src + (int64_t)(r + off) * lds;
    for (int c = threadIdx.x; c < n; c += kT) d[c] = a[c] + b[c];
  } else {
    for (int c = threadIdx.x; c < n; c += kT) d[c] = a[c];
  }
}

__global__ __launch_bounds__(kT) void k_argmax(Params P, const float* logits, int32_t* next) {
  __shared__ unsigned long long red[kT / 64];
  const int b = blockIdx.x;
  const float* x = logits + (int64_t)b * P.V;
  unsigned long long best = 0;
  for (int i = threadIdx.x; i < P.V; i += kT) {
    const unsigned long long k = argmax_key(x[i], (uint32_t)i);
    best = k > best ? k : best;
  }
  best = wave_max_u64(best);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kT / 64; ++w) best = red[w] > best ? red[w] : best;
    best = red[0] > best ? red[0] : best;
    next[b] = (int32_t)(0xFFFFFFFFu - (uint32_t)best);
    if (!(fabsf(argmax_key_value(best)) <= 3.0e38f)) atomicCAS(&P.status[1], ST_OK, ST_NONFINITE);
  }
}

}  // namespace

hipError_t pf_embed(hipStream_t s, const Params& P, const int32_t* tokens, int tok_stride, int B, int c, int p0,
                    float* X) {
  k_embed<<<dim3(B * c), dim3(kT), 0, s>>>(P, tokens, tok_stride, c, p0, X);
  return hipGetLastError();
}

hipError_t pf_add_norm_split(hipStream_t s, const Params& P, float* X, const float* T, int ldt, const uint16_t* gamma,
                             int n, int rstride, int roff, uint16_t* hi, uint16_t* lo) {
  k_add_norm_split<<<dim3(n), dim3(kT), 0, s>>>(P, X, T, ldt, gamma, rstride, roff, hi, lo);
  return hipGetLastError();
}

hipError_t pf_rope_kv(hipStream_t s, const Params& P, int l, float* QKV, int ldq, int B, int c, int p0) {
  k_rope_kv<<<dim3(B * c), dim3(kT), 0, s>>>(P, l, QKV, ldq, c, p0);
  return hipGetLastError();
}

hipError_t pf_prepare(int hd) {
  hipError_t e = hipSuccess;
  if (hd == 64) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attention<64, float>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, attn_lds_bytes(64));
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attention<64, uint16_t>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, attn_lds_bytes(64));
  } else {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attention<128, float>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, attn_lds_bytes(128));
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attention<128, uint16_t>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, attn_lds_bytes(128));
  }
  return e;
}

hipError_t pf_attention(hipStream_t s, const Params& P, int l, const float* QKV, int ldq, int B, int c, int p0,
                        uint16_t* hi, uint16_t* lo) {
  const int G = P.nq / P.nkv, Qb = 64 / G;
  const dim3 grid((c + Qb - 1) / Qb, P.nkv, B);
  if (P.hd == 128 && !P.kv_f32) {  // bf16 cache: the matrix cores
    k_attention_mma<<<grid, dim3(kT), 0, s>>>(P, l, QKV, ldq, c, p0, hi, lo);
  } else if (P.hd == 64) {
    if (P.kv_f32) k_attention<64, float><<<grid, dim3(kT), attn_lds_bytes(64), s>>>(P, l, QKV, ldq, c, p0, hi, lo);
    else k_attention<64, uint16_t><<<grid, dim3(kT), attn_lds_bytes(64), s>>>(P, l, QKV, ldq, c, p0, hi, lo);
  } else {
    if (P.kv_f32) k_attention<128, float><<<grid, dim3(kT), attn_lds_bytes(128), s>>>(P, l, QKV, ldq, c, p0, hi, lo);
    else k_attention<128, uint16_t><<<grid, dim3(kT), attn_lds_bytes(128), s>>>(P, l, QKV, ldq, c, p0, hi, lo);
  }
  return hipGetLastError();
}

hipError_t pf_swiglu_split(hipStream_t s, const Params& P, const float* GU, int rows, uint16_t* hi, uint16_t* lo) {
  k_swiglu_split<<<dim3(rows), dim3(kT), 0, s>>>(P, GU, hi, lo);
  return hipGetLastError();
}

hipError_t pf_fold(hipStream_t s, const float* src, int lds, int off, float* dst, int ldd, int rows, int n) {
  k_fold<<<dim3(rows), dim3(kT), 0, s>>>(src, lds, off, dst, ldd, n);
  return hipGetLastError();
}

hipError_t pf_argmax(hipStream_t s, const Params& P, const float* logits, int B, int32_t* next) {
  k_argmax<<<dim3(B), dim3(kT), 0, s>>>(P, logits, next);
  return hipGetLastError();
}

}  // namespace mk
