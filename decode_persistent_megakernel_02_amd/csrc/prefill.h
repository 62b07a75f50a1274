// Batched prefill: the kernels between the projections (prefill.hip) and their
// launchers.  Rows of a chunk are (sequence b, position p0 + i) for b < B,
// i < c, row r = b c + i; activations are row-major fp32 [rows][width], GEMM
// operands bf16 planes (high part, then low part: v = hi + lo to about 2^-16
// relative), row-major [rows][K].
#pragma once
#include <hip/hip_runtime.h>

#include "mk_internal.h"

namespace mk {

constexpr int kPrefillStack = 512;  // up to this many rows a projection is one GEMM over both operand parts

// X[r] = embedding row of the token of row r (tokens[b tok_stride + p0 + i]).
hipError_t pf_embed(hipStream_t s, const Params& P, const int32_t* tokens, int tok_stride, int B, int c, int p0,
                    float* X);
// For n output rows o (source row o * rstride + roff): X[src] += T[src] when T
// is given (row stride ldt), then the RMSNorm of X[src] times gamma, split into
// hi[o], lo[o] (row stride H).
hipError_t pf_add_norm_split(hipStream_t s, const Params& P, float* X, const float* T, int ldt, const uint16_t* gamma,
                             int n, int rstride, int roff, uint16_t* hi, uint16_t* lo);
// Rotates the query and key heads of each row's [q | k | v] (row stride ldq)
// by its position and appends k and v to layer l's cache.
hipError_t pf_rope_kv(hipStream_t s, const Params& P, int l, float* QKV, int ldq, int B, int c, int p0);
// Causal attention of each row's query heads over its sequence's cache
// positions 0 .. p (layer l), written as hi/lo planes [rows][nq hd].
hipError_t pf_attention(hipStream_t s, const Params& P, int l, const float* QKV, int ldq, int B, int c, int p0,
                        uint16_t* hi, uint16_t* lo);
// h = silu(gate) * up for GU = [gate | up] (row stride 2F), as hi/lo planes [rows][F].
hipError_t pf_swiglu_split(hipStream_t s, const Params& P, const float* GU, int rows, uint16_t* hi, uint16_t* lo);
// dst[r][c] = src[r][c] + src[off + r][c] (off 0: a copy) for r < rows, c < n;
// row strides lds, ldd; dst may be src.
hipError_t pf_fold(hipStream_t s, const float* src, int lds, int off, float* dst, int ldd, int rows, int n);
// next[b] = first index of the largest of logits[b][0, V).
hipError_t pf_argmax(hipStream_t s, const Params& P, const float* logits, int B, int32_t* next);
// LDS bytes of the attention kernel by head dim; registers its limit.
hipError_t pf_prepare(int hd);

}  // namespace mk
