// Latent cache write for gfx950: each token's 512 compressed dims (kv_c) and
// 64 RoPE dims (k_pe) go, concatenated, into its pool slot, the step that
// feeds the decode path (vLLM pull request 57942, Details: the KV-cache write
// of decode). Each source is read at its own dtype and converted; nothing is
// reinterpreted (the same page's review thread finds an fp32 k_pe written as
// if it were bf16, leaving garbage RoPE columns).
//
// General form: one wave per token; lane l handles elements l, l + 64, ... of
// the 576, so every load and store of a wave covers 64 consecutive elements.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "kernel_args.h"

namespace mla {
namespace {

constexpr int kRow = 576, kNope = 512;

__device__ __forceinline__ float load_src(const void* base, int dtype, int64_t i) {
  if (dtype == 0) return (float)((const __bf16*)base)[i];
  if (dtype == 1) return (float)((const _Float16*)base)[i];
  return ((const float*)base)[i];
}

// fp32 -> OCP e4m3fn: NaN -> 0x7F, saturate to +-448, then the hardware's
// round-to-nearest-even conversion (the sign of a zero result is kept).
__device__ __forceinline__ uint8_t to_e4m3fn(float v) {
  if (__builtin_isnan(v)) return 0x7F;
  v = fminf(fmaxf(v, -448.0f), 448.0f);
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xFF);
}

// x / s rounded to nearest, from r = 1 / s (itself correctly rounded, one
// division per thread) and one fused correction: by Markstein's theorem
// (IBM J. Res. Dev. 34(1), 1990), when r is the correctly rounded reciprocal
// and q0 lies within one ulp of x / s, q0 + r (x - q0 s) rounded once is the
// correctly rounded quotient, for quotients in the normal range. Zero, tiny
// (below 2^-100), saturating (above 448) and non-finite quotients keep q0:
// the e4m3fn encoding maps them to the same code as the exact quotient.
__device__ __forceinline__ float div_rn(float x, float s, float r) {
  const float q0 = x * r;
  const float rem = __builtin_fmaf(-q0, s, x);   // exact
  const float q1 = __builtin_fmaf(rem, r, q0);
  const float aq = __builtin_fabsf(q0);
  return (aq >= 0x1p-100f && aq <= 448.0f) ? q1 : q0;
}
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.tokens) return;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_slots) return;   // padding token, or out of the pool
  const int lane = threadIdx.x & 63;
  const float scale = a.kv_scale ? *a.kv_scale : 1.0f;
  const float rscale = 1.0f / scale;
  for (int e = lane; e < kRow; e += 64) {
    const float x = e < kNope ? load_src(a.kv_c, a.kv_c_dtype, (int64_t)t * a.kv_c_stride + e)
                              : load_src(a.k_pe, a.k_pe_dtype, (int64_t)t * a.k_pe_stride + e - kNope);
    const int64_t o = slot * kRow + e;
    if (a.kv_fp8) ((uint8_t*)a.pool)[o] = to_e4m3fn(div_rn(x, scale, rscale));
    else ((__bf16*)a.pool)[o] = (__bf16)x;                           // round to nearest even
  }
}

// Vector form, for 16-byte aligned source rows and pool (bf16 pool): thread
// c converts elements 8 p .. 8 p + 7 of token c / 72 (p = c mod 72; p < 64 is
// kv_c), with one 16-byte (32 for fp32) load and one 16-byte store. Same
// conversions as above.
template <int SRC>
__device__ __forceinline__ void load8(const void* base, int64_t i, float (&x)[8]) {
  if constexpr (SRC == 0) {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    const v8 v = *(const v8*)((const __bf16*)base + i);
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = (float)v[k];
  } else if constexpr (SRC == 1) {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    const v8 v = *(const v8*)((const _Float16*)base + i);
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = (float)v[k];
  } else {
    typedef float v4 __attribute__((ext_vector_type(4)));
    const v4 a = *(const v4*)((const float*)base + i);
    const v4 b = *(const v4*)((const float*)base + i + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) { x[k] = a[k]; x[k + 4] = b[k]; }
  }
}

template <int SRC_C, int SRC_PE>
__global__ __launch_bounds__(256) void cache_write_bf16_vec_kernel(CacheWriteArgs a) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= (int64_t)a.tokens * 72) return;
  const int t = (int)(c / 72), p = (int)(c - (int64_t)t * 72);
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_slots) return;
  float x[8];
  if (p < 64) load8<SRC_C>(a.kv_c, (int64_t)t * a.kv_c_stride + 8 * p, x);
  else load8<SRC_PE>(a.k_pe, (int64_t)t * a.k_pe_stride + 8 * (p - 64), x);
  const int64_t o = slot * kRow + 8 * p;
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  v8 v;
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = (__bf16)x[k];
  *(v8*)((__bf16*)a.pool + o) = v;
}

// fp8 pool: thread c converts elements 16 p .. 16 p + 15 of token c / 36
// (p = c mod 36; p < 32 is kv_c), two 8-element loads and one 16-byte store
// (with 8 elements and 8-byte stores per thread the write took 21% longer).
template <int SRC_C, int SRC_PE>
__global__ __launch_bounds__(256) void cache_write_fp8x16_kernel(CacheWriteArgs a) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= (int64_t)a.tokens * 36) return;
  const int t = (int)(c / 36), p = (int)(c - (int64_t)t * 36);
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_slots) return;
  float x[2][8];
  if (p < 32) {
    load8<SRC_C>(a.kv_c, (int64_t)t * a.kv_c_stride + 16 * p, x[0]);
    load8<SRC_C>(a.kv_c, (int64_t)t * a.kv_c_stride + 16 * p + 8, x[1]);
  } else {
    load8<SRC_PE>(a.k_pe, (int64_t)t * a.k_pe_stride + 16 * (p - 32), x[0]);
    load8<SRC_PE>(a.k_pe, (int64_t)t * a.k_pe_stride + 16 * (p - 32) + 8, x[1]);
  }
  const float scale = a.kv_scale ? *a.kv_scale : 1.0f;
  const float rscale = 1.0f / scale;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < 16; ++k)
    w[k >> 2] |= (uint32_t)to_e4m3fn(div_rn(x[k >> 3][k & 7], scale, rscale)) << (8 * (k & 3));
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  *(u4*)((uint8_t*)a.pool + slot * kRow + 16 * p) = u4{w[0], w[1], w[2], w[3]};
}

template <int SRC_C>
const void* fp8x16_kernel_for(int src_pe) {
  if (src_pe == 0) return (const void*)cache_write_fp8x16_kernel<SRC_C, 0>;
  if (src_pe == 1) return (const void*)cache_write_fp8x16_kernel<SRC_C, 1>;
  return (const void*)cache_write_fp8x16_kernel<SRC_C, 2>;
}

template <int SRC_C>
const void* vec_kernel_for(int src_pe) {
  if (src_pe == 0) return (const void*)cache_write_bf16_vec_kernel<SRC_C, 0>;
  if (src_pe == 1) return (const void*)cache_write_bf16_vec_kernel<SRC_C, 1>;
  return (const void*)cache_write_bf16_vec_kernel<SRC_C, 2>;
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, bool vec, hipStream_t st) {
  void* args[] = {(void*)&a};
  if (vec && a.kv_fp8) {
    const void* fn = a.kv_c_dtype == 0 ? fp8x16_kernel_for<0>(a.k_pe_dtype)
                     : a.kv_c_dtype == 1 ? fp8x16_kernel_for<1>(a.k_pe_dtype) : fp8x16_kernel_for<2>(a.k_pe_dtype);
    const int64_t threads = (int64_t)a.tokens * 36;
    return hipLaunchKernel(fn, dim3((unsigned)((threads + 255) / 256)), dim3(256), args, 0, st);
  }
  if (vec) {
    const void* fn = a.kv_c_dtype == 0 ? vec_kernel_for<0>(a.k_pe_dtype)
                     : a.kv_c_dtype == 1 ? vec_kernel_for<1>(a.k_pe_dtype) : vec_kernel_for<2>(a.k_pe_dtype);
    const int64_t threads = (int64_t)a.tokens * 72;
    return hipLaunchKernel(fn, dim3((unsigned)((threads + 255) / 256)), dim3(256), args, 0, st);
  }
  return hipLaunchKernel((const void*)cache_write_kernel, dim3((a.tokens + 3) / 4), dim3(256), args, 0, st);
}

}  // namespace mla
