// Split-merge kernels for CDNA4 (gfx950): the log-sum-exp merge of a row's
// split partials ([DSV4] Tuned ASM FP8 decode with split plans, ATOM pull
// request 2462, Dependencies: split and merge), the merge of
// decode-context-parallel shard results (ATOM pull request 2760, Problem), and
// a fill kernel for the workspace's split counters.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "device_common.h"
#include "kernel_args.h"

namespace mla {
namespace {

using namespace dev;

constexpr int kDV = 512;
constexpr int kMergeLanes = 4;   // splits per lane: n <= 256

// ---------------------------------------------------------------------------
// Split merge: one block of four waves per (request row b, query token i,
// heads 4 j .. 4 j + 3) of a row with n > 1 splits (n <= 256). Lane l of a
// wave reads LSE_k for k = l + 64 i and the wave reduces max and sum. With n <= 8 splits each wave
// merges one head, all n partials' loads in flight at once; with more, the
// four waves take every fourth split of one head at a time and add up in
// LDS. A lane owns 8 output columns.
// Weights of the n partials of one (token, head): lane l gets
// exp(LSE_k - LSE) for its splits k; returns false (and writes O = 0, LSE = -inf) when every
// split is empty.
__device__ __forceinline__ bool merge_weights(const MergeArgs& a, int64_t base, int64_t stride, int n,
                                              int lane, int64_t orow, float (&wk)[kMergeLanes], float& lse,
                                              bool writer) {
  // Lane l holds split k = l + 64 i in slot i (up to 256 splits).
  float lk[kMergeLanes];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMergeLanes; ++i) {
    const int k = lane + 64 * i;
    lk[i] = k < n ? a.ws_lse[base + k * stride] : -INFINITY;
    mx = fmaxf(mx, lk[i]);
  }
  mx = wave_max(mx);
  if (mx == -INFINITY) {
    if (writer) {
      *(u32x4*)(a.o + orow * kDV + lane * 8) = u32x4{0u, 0u, 0u, 0u};
      if (lane == 0) a.lse[orow] = -INFINITY;
    }
    return false;
  }
  const float kLog2e = 1.44269504088896340736f;
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < kMergeLanes; ++i) {
    wk[i] = lk[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lk[i] - mx) * kLog2e);
    part += wk[i];
  }
  const float tot = wave_sum(part);
#pragma unroll
  for (int i = 0; i < kMergeLanes; ++i) wk[i] /= tot;
  lse = mx + __log2f(tot) * kLn2;
  return true;
}

// 8 columns of a bf16 partial O as fp32.
__device__ __forceinline__ void load_partial(const uint16_t* p, f32x4 (&v)[2]) {
  const bf16x8 x = *(const bf16x8*)p;
  v[0] = f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
  v[1] = f32x4{(float)x[4], (float)x[5], (float)x[6], (float)x[7]};
}

// Weight of split k (wave-uniform k < 256) from merge_weights' registers.
__device__ __forceinline__ float weight_of(const float (&wk)[kMergeLanes], int k) {
  const int i = k >> 6;   // uniform
  const float v = i == 0 ? wk[0] : i == 1 ? wk[1] : i == 2 ? wk[2] : wk[3];
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), k & 63));
}

__device__ __forceinline__ void store_row(const MergeArgs& a, int64_t orow, int lane, f32x4 acc0, f32x4 acc1,
                                          float lse) {
  *(bf16x8*)(a.o + orow * kDV + lane * 8) =
      bf16x8{(__bf16)acc0[0], (__bf16)acc0[1], (__bf16)acc0[2], (__bf16)acc0[3],
             (__bf16)acc1[0], (__bf16)acc1[1], (__bf16)acc1[2], (__bf16)acc1[3]};
  if (lane == 0) a.lse[orow] = lse;
}

__global__ __launch_bounds__(kBlockThreads) void merge_kernel(MergeArgs a) {
  __shared__ f32x4 part[kBlockThreads / 64 - 1][64][2];
  constexpr int kW = kBlockThreads / 64;
  const int hgroups = (a.heads + kW - 1) / kW;
  const int hg = blockIdx.x % hgroups;
  const int bi = blockIdx.x / hgroups;
  const int b = bi / a.q_len_max;
  const int i = bi - b * a.q_len_max;
  const int s0 = a.plan[a.off_split_indptr + b];
  const int n = a.plan[a.off_split_indptr + b + 1] - s0;
  if (n <= a.skip_upto) return;   // unsplit, or merged in the decode kernel
  const int q0 = a.qo_indptr[b];
  if (i >= a.qo_indptr[b + 1] - q0) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int part0 = a.plan[a.off_split_part + s0];
  const int64_t stride = (int64_t)a.q_len_max * a.heads;   // partial slots are consecutive

  if (n <= 8) {   // one wave per head (uniform over the block: n is the row's)
    const int h = hg * kW + w;
    if (h >= a.heads) return;
    const int64_t base = ((int64_t)part0 * a.q_len_max + i) * a.heads + h;
    const int64_t orow = (int64_t)(q0 + i) * a.heads + h;
    float wk[kMergeLanes], lse;
    if (!merge_weights(a, base, stride, n, lane, orow, wk, lse, true)) return;
    const uint16_t* src = a.ws_o + base * kDV + lane * 8;
    f32x4 v[8][2];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < n) load_partial(src + k * stride * kDV, v[k]);
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < n) {
        const float c = weight_of(wk, k);
        acc0 += c * v[k][0];   // an empty split's partial is 0 and its weight 0
        acc1 += c * v[k][1];
      }
    store_row(a, orow, lane, acc0, acc1, lse);
    return;
  }

  for (int hh = 0; hh < kW; ++hh) {   // four waves per head, one head at a time
    const int h = hg * kW + hh;
    if (h >= a.heads) break;          // uniform
    const int64_t base = ((int64_t)part0 * a.q_len_max + i) * a.heads + h;
    const int64_t orow = (int64_t)(q0 + i) * a.heads + h;
    float wk[kMergeLanes], lse;
    if (!merge_weights(a, base, stride, n, lane, orow, wk, lse, w == 0)) continue;   // uniform
    const uint16_t* src = a.ws_o + base * kDV + lane * 8;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = w; k0 < n; k0 += 8 * kW) {
      f32x4 v[8][2];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u * kW;
        if (k < n) load_partial(src + k * stride * kDV, v[u]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u * kW;
        if (k < n) {
          const float c = weight_of(wk, k);
          acc0 += c * v[u][0];
          acc1 += c * v[u][1];
        }
      }
    }
    if (w > 0) {
      part[w - 1][lane][0] = acc0;
      part[w - 1][lane][1] = acc1;
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int j = 0; j < kW - 1; ++j) {
        acc0 += part[j][lane][0];
        acc1 += part[j][lane][1];
      }
      store_row(a, orow, lane, acc0, acc1, lse);
    }
    __syncthreads();   // part[] is reused for the next head
  }
}

// ---------------------------------------------------------------------------
// Merge of decode-context-parallel shard outputs: one wave per (token, head)
// row; lane k < world reads LSE_k, the wave reduces max and sum, and every
// lane accumulates 8 columns of the weighted bf16 shard outputs (a shard with
// no visible key has O = 0 and weight 0).
__global__ __launch_bounds__(kBlockThreads) void shard_merge_kernel(ShardMergeArgs a) {
  const int row = blockIdx.x * (kBlockThreads / 64) + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int lane = threadIdx.x & 63;
  const float lk = lane < a.world ? a.lse_parts[(int64_t)lane * a.rows + row] : -INFINITY;
  const float mx = wave_max(lk);
  uint16_t* dst = a.o + (int64_t)row * kDV + lane * 8;
  if (mx == -INFINITY) {   // no shard sees a key
    *(u32x4*)dst = u32x4{0u, 0u, 0u, 0u};
    if (lane == 0) a.lse[row] = -INFINITY;
    return;
  }
  const float kLog2e = 1.44269504088896340736f;
  const float ek = lk == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lk - mx) * kLog2e);
  const float tot = wave_sum(ek);
  const float wk = ek / tot;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k = 0; k < a.world; ++k) {
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wk), k));
    const bf16x8 v = *(const bf16x8*)(a.o_parts + ((int64_t)k * a.rows + row) * kDV + lane * 8);
    acc0 += c * f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    acc1 += c * f32x4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
  }
  *(bf16x8*)dst = bf16x8{(__bf16)acc0[0], (__bf16)acc0[1], (__bf16)acc0[2], (__bf16)acc0[3],
                         (__bf16)acc1[0], (__bf16)acc1[1], (__bf16)acc1[2], (__bf16)acc1[3]};
  if (lane == 0) a.lse[row] = mx + __log2f(tot) * kLn2;
}

// Fills a buffer with zeros (the workspace's split counters); a kernel, not a
// memset, so that it may sit in a captured graph.
__global__ __launch_bounds__(256) void zero_kernel(uint32_t* p, int32_t words) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < words) p[i] = 0u;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int rows, int heads, int q_len_max, hipStream_t st) {
  void* args[] = {(void*)&a};
  constexpr int kW = kBlockThreads / 64;
  dim3 grid(rows * q_len_max * ((heads + kW - 1) / kW));
  return hipLaunchKernel((const void*)merge_kernel, grid, dim3(kBlockThreads), args, 0, st);
}

hipError_t launch_zero(uint32_t* p, int32_t words, hipStream_t st) {
  void* args[] = {(void*)&p, (void*)&words};
  return hipLaunchKernel((const void*)zero_kernel, dim3((words + 255) / 256), dim3(256), args, 0, st);
}

hipError_t launch_shard_merge(const ShardMergeArgs& a, hipStream_t st) {
  void* args[] = {(void*)&a};
  const int per = kBlockThreads / 64;
  return hipLaunchKernel((const void*)shard_merge_kernel, dim3((a.rows + per - 1) / per),
                         dim3(kBlockThreads), args, 0, st);
}

}  // namespace mla
