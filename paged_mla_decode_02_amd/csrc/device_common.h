// Device helpers shared by the library's HIP sources (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mla {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// 16-byte (and 4-byte) direct-to-LDS loads: lane l's data lands at LDS byte
// address lds_addr + 16 l (4 l). Inline assembly keeps them out of the
// compiler's wait-count tracking (it would otherwise wait for the next tiles'
// loads before every LDS read of the current one); completion is awaited
// explicitly with wait_vm before the barrier that publishes a tile. The
// compiler never uses M0 in these kernels (checked on the generated code), so
// setting it here is safe. The LDS address is wave-uniform by construction;
// readfirstlane makes that explicit for the scalar operand.
__device__ __forceinline__ void dma16_sbase(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(sbase) : "memory");
}
__device__ __forceinline__ void dma16_vaddr(const void* vaddr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(vaddr) : "memory");
}
__device__ __forceinline__ void dma4_vaddr(const void* vaddr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(vaddr) : "memory");
}

// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N> __device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void wait_vm_all() { wait_vm<0>(); }

__device__ __forceinline__ uint32_t lds_addr_of(const lds_u8* p) { return (uint32_t)(uintptr_t)p; }

// A copy of v the compiler cannot see through: values derived from it inside
// a loop are recomputed there (a few VALU ops) instead of being hoisted out of
// the loop and kept live.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// The lane id, computed afresh where it is used (two VALU ops the compiler
// can neither hoist nor share): a lane id kept live across the item loop is
// a spill candidate, and a reload's wait there also waits for every tile
// load in flight.
__device__ __forceinline__ int lane_now() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// v of lane src (0..63) of the wave; no lane id of its own (unlike __shfl).
__device__ __forceinline__ int bpermute(int src, int v) {
  return __builtin_amdgcn_ds_bpermute(src << 2, v);
}

// The same for a wave-uniform value kept in a scalar register.
__device__ __forceinline__ int opaque_s(int v) {
  asm volatile("" : "+s"(v));
  return v;
}

// n / d for 0 <= n < 2^20 and 1 <= d <= 2^16: a float estimate from the
// hardware reciprocal (relative error below 2^-22, so the estimate is within
// one of the quotient) corrected by one remainder test each way. Nothing of
// it is hoisted out of a loop, unlike the compiler's division sequence.
__device__ __forceinline__ int div_small(int n, int d) {
  int q = (int)((float)n * __builtin_amdgcn_rcpf((float)d));
  const int r = n - q * d;
  q += r >= d ? 1 : 0;
  q -= r < 0 ? 1 : 0;
  return q;
}

template <typename T> __device__ __forceinline__ T lds_load(const lds_u8* base, int off) {
  return *(const __attribute__((address_space(3))) T*)(base + off);
}
template <typename T> __device__ __forceinline__ void lds_store(lds_u8* base, int off, T v) {
  *(__attribute__((address_space(3))) T*)(base + off) = v;
}

// 4 fp8 (OCP e4m3fn) bytes -> 4 bf16, exact.
__device__ __forceinline__ bf16x4 fp8x4_to_bf16(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return bf16x4{lo[0], lo[1], hi[0], hi[1]};
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// max / sum of v over lanes l and l ^ 32 (one v_permlane32_swap).
__device__ __forceinline__ float half_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float half_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Reductions over the four 16-lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48):
// v_permlane32_swap and v_permlane16_swap exchange halves and odd/even
// 16-lane rows between two registers, so each step is one VALU swap.
__device__ __forceinline__ float group_max(float v) {
  v = half_max(v);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float v) {
  v = half_sum(v);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_max(float v) {
  v = group_max(v);
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}
// Minimum over the wave without a lane id: lanes l ^ 16 .. l ^ 1 inside each
// 32-lane half by ds_swizzle (bit mode: offset = and 0x1f | xor << 10), then
// the two halves by v_permlane32_swap.
__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, __builtin_amdgcn_ds_swizzle(v, 0x1f | (16 << 10)));
  v = min(v, __builtin_amdgcn_ds_swizzle(v, 0x1f | (8 << 10)));
  v = min(v, __builtin_amdgcn_ds_swizzle(v, 0x1f | (4 << 10)));
  v = min(v, __builtin_amdgcn_ds_swizzle(v, 0x1f | (2 << 10)));
  v = min(v, __builtin_amdgcn_ds_swizzle(v, 0x1f | (1 << 10)));
  const auto a = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return min((int)a[0], (int)a[1]);
}
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum(v);
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

}  // namespace dev
}  // namespace mla
