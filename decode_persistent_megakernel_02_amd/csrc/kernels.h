// Declarations of the device entry points (defined in kernels.hip).
#pragma once
#include <hip/hip_runtime.h>

#include "mk_internal.h"

namespace mk {
// megakernel instances (mega.hip): mk_mega_<x|n>_<head_dim>_<f32|bf16>_g<query heads per KV head>
#define MK_MEGA_DECL(X, HD, KN, G) extern "C" __global__ void mk_mega_##X##_##HD##_##KN##_g##G(Params P, MegaBufs M, Step S, int pf);
#define MK_MEGA_DECL_G(X, HD, KN) MK_MEGA_DECL(X, HD, KN, 1) MK_MEGA_DECL(X, HD, KN, 2) MK_MEGA_DECL(X, HD, KN, 4) MK_MEGA_DECL(X, HD, KN, 8)
MK_MEGA_DECL_G(n, 64, f32) MK_MEGA_DECL_G(n, 64, bf16) MK_MEGA_DECL_G(n, 128, f32) MK_MEGA_DECL_G(n, 128, bf16)
MK_MEGA_DECL(x, 64, f32, 4) MK_MEGA_DECL(x, 64, bf16, 4) MK_MEGA_DECL(x, 128, f32, 4) MK_MEGA_DECL(x, 128, bf16, 4)
#undef MK_MEGA_DECL_G
#undef MK_MEGA_DECL
int mega_lds_bytes(int H, int nq, int nkv, int hd, int F, int* page_floats);  // megakernel LDS by shape
#define MK_ATTN_DECL(KN, GQ)                                                                                 \
  extern "C" __global__ void mk_op_attn_split_##KN##_g##GQ(Params P, const Step* S, int layer, int fuse_merge); \
  extern "C" __global__ void mk_op_attn_full_##KN##_g##GQ(Params P, const Step* S, int layer);
#define MK_ATTN_DECL_G(KN) MK_ATTN_DECL(KN, 0) MK_ATTN_DECL(KN, 1) MK_ATTN_DECL(KN, 2) MK_ATTN_DECL(KN, 4) MK_ATTN_DECL(KN, 8)
MK_ATTN_DECL_G(f32)
MK_ATTN_DECL_G(bf16)
#undef MK_ATTN_DECL_G
#undef MK_ATTN_DECL
extern "C" __global__ void mk_op_attn_merge(Params P, const Step* S, int layer);
extern "C" __global__ void mk_set_step(Step* dst, Step s);
#define MK_OP_DECL(name) extern "C" __global__ void name(Params P, const Step* S, OpArgs A, int pf, int sf);
MK_OP_DECL(mk_op_qkv)
MK_OP_DECL(mk_op_o)
MK_OP_DECL(mk_op_gu)
MK_OP_DECL(mk_op_down)
MK_OP_DECL(mk_op_lm)
MK_OP_DECL(mk_op_argmax)
MK_OP_DECL(mk_op_qkv_x)
MK_OP_DECL(mk_op_o_x)
MK_OP_DECL(mk_op_gu_x)
MK_OP_DECL(mk_op_down_x)
MK_OP_DECL(mk_op_lm_x)
#undef MK_OP_DECL
// batched path (batched.hip)
#define MK_BGEMM_DECL(name) extern "C" __global__ void name(Params P, const Step* S, int layer);
#define MK_BGEMM_DECL_ALL(op)                                                                      \
  MK_BGEMM_DECL(mk_b_##op##_b1) MK_BGEMM_DECL(mk_b_##op##_b2) MK_BGEMM_DECL(mk_b_##op##_b4)       \
  MK_BGEMM_DECL(mk_b_##op##_b1_t) MK_BGEMM_DECL(mk_b_##op##_b2_t) MK_BGEMM_DECL(mk_b_##op##_b4_t) \
  MK_BGEMM_DECL(mk_b_##op##_b4_g2) MK_BGEMM_DECL(mk_b_##op##_b4_t_g2)
MK_BGEMM_DECL_ALL(qkv) MK_BGEMM_DECL_ALL(o) MK_BGEMM_DECL_ALL(gu) MK_BGEMM_DECL_ALL(down) MK_BGEMM_DECL_ALL(lm)
#undef MK_BGEMM_DECL_ALL
#undef MK_BGEMM_DECL
extern "C" __global__ void mk_b_fin_qkv(Params P, const Step* S, int layer, int ks);
extern "C" __global__ void mk_b_fin_o(Params P, const Step* S, int layer, int ks);
extern "C" __global__ void mk_b_fin_gu(Params P, const Step* S, int layer, int ks);
extern "C" __global__ void mk_b_fin_down(Params P, const Step* S, int layer, int ks);
int b_lds_bytes(int bt);  // LDS of the batched projection kernels by batch tiles
constexpr int kBChunkCols[5] = {0, 256, 128, 128, 128};  // activation chunk width by batch tiles
extern "C" __global__ void mk_b_norm(Params P, const Step* S, int layer, int kind);
extern "C" __global__ void mk_b_argmax(Params P, const Step* S);
extern "C" __global__ void mk_t_bgemm_kernel(const uint16_t* W, const uint16_t* A, float* Y, int N, int K, int B,
                                             int tiled);
extern "C" __global__ void mk_tile_kernel(const uint16_t* src, uint16_t* dst, int64_t N, int64_t K);
extern "C" __global__ void mk_fill_u32(uint32_t* p, int64_t n, uint32_t v);
extern "C" __global__ void mk_t_gemv_kernel(const uint16_t* W, const float* x, float* y, int N, int K);
extern "C" __global__ void mk_t_rmsnorm_kernel(const float* x, const uint16_t* gamma, float eps, float* y, int n);
extern "C" __global__ void mk_t_attn_partial_kernel(const float* q, const void* k, const void* v, int64_t head_stride,
                                                    int nq, int nkv, int hd, int T, int split, int nsplit, int kv_f32,
                                                    float* part);
extern "C" __global__ void mk_t_attn_merge_kernel(const float* part, int nq, int nkv, int hd, int T, int split,
                                                  int nsplit, float* o);
extern "C" __global__ void mk_t_argmax_kernel(const float* x, int n, unsigned long long* slot);
extern "C" __global__ void mk_t_argmax_final(const unsigned long long* slot, int32_t* out);
hipError_t launch_stream_read(const void* src, int64_t nvec, int wgs, int loads, uint32_t* sink, hipStream_t st);
}  // namespace mk
