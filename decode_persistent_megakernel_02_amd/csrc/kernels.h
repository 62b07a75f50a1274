// Declarations of the device entry points (defined in kernels.hip).
#pragma once
#include <hip/hip_runtime.h>

#include "mk_internal.h"

namespace mk {
extern "C" __global__ void mk_persistent(Params P, Step S, int page_floats, int scratch_floats);
extern "C" __global__ void mk_stage(Params P, Step S, const Task* tasks, int count, int page_floats, int scratch_floats);
extern "C" __global__ void mk_fill_u32(uint32_t* p, int64_t n, uint32_t v);
extern "C" __global__ void mk_t_gemv_kernel(const uint16_t* W, const float* x, float* y, int N, int K);
extern "C" __global__ void mk_t_rmsnorm_kernel(const float* x, const uint16_t* gamma, float eps, float* y, int n);
extern "C" __global__ void mk_t_attn_partial_kernel(const float* q, const uint16_t* k, const uint16_t* v,
                                                    int64_t head_stride, int nq, int nkv, int hd, int T, int split,
                                                    int nsplit, float* part);
extern "C" __global__ void mk_t_attn_merge_kernel(const float* part, int nq, int nkv, int hd, int T, int split,
                                                  int nsplit, float* o);
extern "C" __global__ void mk_t_argmax_kernel(const float* x, int n, unsigned long long* slot);
extern "C" __global__ void mk_t_argmax_final(const unsigned long long* slot, int32_t* out);
}  // namespace mk
