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
constexpr int kChunkWide = 16;   // splits whose loads a lane of merge_wide_kernel has in flight at once

// ---------------------------------------------------------------------------
// Split merge: one block of four waves per (request row b, query token i,
// heads 4 j .. 4 j + 3) of a row with n > 1 splits; each wave merges one
// head, a lane owning 8 of the 512 output columns. The split partials are
// merged by log-sum-exp, online, in chunks: a chunk's partial-O loads and LSE
// loads are issued together (the LSE addresses are wave-uniform), so a chunk
// costs one memory round trip, and the running (max, sum, O) are rescaled
// when a chunk raises the max. The chunk size C (2, 4 or 8 splits) is the
// smallest that covers the plan's largest split count up to 8, so a row takes
// ceil(n / C) round trips, the four heads of a block in parallel, and a wave
// holds no more registers than its chunk needs (the waves in flight per SIMD
// grow as the chunk shrinks).
struct MergeState {
  float m, l;       // running max of LSE_k, and sum of exp(LSE_k - m)
  f32x4 acc0, acc1; // sum of exp(LSE_k - m) O_k over this lane's 8 columns
};

// Splits k = k0 + j, j < C, k < n, of the partial rows at `src` (this lane's
// 8 columns) and `lse_base` (uniform), folded into st.
template <int C>
__device__ __forceinline__ void merge_chunk(const uint16_t* src, const float* lse_base, int64_t stride, int k0,
                                            int n, MergeState& st) {
  bf16x8 v[C];
  float lk[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int k = k0 + j;
    if (k < n) {
      v[j] = *(const bf16x8*)(src + (int64_t)k * stride * kDV);
      lk[j] = lse_base[(int64_t)k * stride];
    } else {
      lk[j] = -INFINITY;
    }
  }
  float cm = lk[0];
#pragma unroll
  for (int j = 1; j < C; ++j) cm = fmaxf(cm, lk[j]);
  if (cm == -INFINITY) return;   // every split of the chunk is empty (uniform)
  const float mnew = fmaxf(st.m, cm);
  if (mnew > st.m) {   // uniform
    const float r = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((st.m - mnew) * kLog2e);
    st.l *= r;
    st.acc0 *= r;
    st.acc1 *= r;
    st.m = mnew;
  }
#pragma unroll
  for (int j = 0; j < C; ++j) {
    if (lk[j] != -INFINITY) {   // an empty split's partial O is 0 and carries no weight
      const float c = __builtin_amdgcn_exp2f((lk[j] - mnew) * kLog2e);
      st.l += c;
      st.acc0 += c * f32x4{(float)v[j][0], (float)v[j][1], (float)v[j][2], (float)v[j][3]};
      st.acc1 += c * f32x4{(float)v[j][4], (float)v[j][5], (float)v[j][6], (float)v[j][7]};
    }
  }
}

// O = acc / l (bf16) and LSE = m + ln l, or O = 0 and LSE = -inf when no
// split saw a key.
__device__ __forceinline__ void store_merged(const MergeArgs& a, int64_t orow, int lane, const MergeState& st) {
  uint16_t* dst = a.o + orow * kDV + lane * 8;
  if (st.m == -INFINITY) {
    *(u32x4*)dst = u32x4{0u, 0u, 0u, 0u};
    if (lane == 0) a.lse[orow] = -INFINITY;
    return;
  }
  const float inv = 1.0f / st.l;
  const f32x4 x0 = st.acc0 * inv, x1 = st.acc1 * inv;
  *(bf16x8*)dst = bf16x8{(__bf16)x0[0], (__bf16)x0[1], (__bf16)x0[2], (__bf16)x0[3],
                         (__bf16)x1[0], (__bf16)x1[1], (__bf16)x1[2], (__bf16)x1[3]};
  if (lane == 0) a.lse[orow] = st.m + __log2f(st.l) * kLn2;
}

template <int C>
__global__ __launch_bounds__(kBlockThreads) void merge_kernel(MergeArgs a) {
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
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = hg * kW + w;
  if (h >= a.heads) return;
  const int part0 = a.plan[a.off_split_part + s0];
  const int64_t stride = (int64_t)a.q_len_max * a.heads;   // partial slots are consecutive
  const int64_t base = ((int64_t)part0 * a.q_len_max + i) * a.heads + h;
  MergeState st{-INFINITY, 0.f, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  // (uniform over the block: n is the row's) A row within one chunk takes it
  // outside the loop: the chunk at the constant offset 0 compiled inside the
  // loop made the verify merge 40% slower.
  if (n <= C) {
    merge_chunk<C>(a.ws_o + base * kDV + lane * 8, a.ws_lse + base, stride, 0, n, st);
  } else {
    for (int k0 = 0; k0 < n; k0 += C)
      merge_chunk<C>(a.ws_o + base * kDV + lane * 8, a.ws_lse + base, stride, k0, n, st);
  }
  store_merged(a, (int64_t)(q0 + i) * a.heads + h, lane, st);
}

// Rows with many splits (long rows cut over many compute units): one block of
// eight waves per (request row b, query token i, head h). Wave w folds chunks
// w, w + 8, w + 16, ... of 16 splits, so up to 128 splits of a row are in
// flight at once, and the eight running states are then combined through LDS
// (each rescaled to the largest max) by wave 0, which stores the row.
constexpr int kWideThreads = 512;
__global__ __launch_bounds__(kWideThreads) void merge_wide_kernel(MergeArgs a) {
  constexpr int kW = kWideThreads / 64;
  __shared__ f32x4 acc_s[kW][2][64];
  __shared__ float ml_s[kW][2];
  const int h = blockIdx.x % a.heads;
  const int bi = blockIdx.x / a.heads;
  const int b = bi / a.q_len_max;
  const int i = bi - b * a.q_len_max;
  const int s0 = a.plan[a.off_split_indptr + b];
  const int n = a.plan[a.off_split_indptr + b + 1] - s0;
  if (n <= a.skip_upto) return;   // unsplit, or merged in the decode kernel (uniform)
  const int q0 = a.qo_indptr[b];
  if (i >= a.qo_indptr[b + 1] - q0) return;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part0 = a.plan[a.off_split_part + s0];
  const int64_t stride = (int64_t)a.q_len_max * a.heads;   // partial slots are consecutive
  const int64_t base = ((int64_t)part0 * a.q_len_max + i) * a.heads + h;
  MergeState st{-INFINITY, 0.f, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  // (the first chunk outside the loop, as in merge_kernel: 11% faster on long
  // context)
  if (kChunkWide * w < n) {
    merge_chunk<kChunkWide>(a.ws_o + base * kDV + lane * 8, a.ws_lse + base, stride, kChunkWide * w, n, st);
    for (int k0 = kChunkWide * (w + kW); k0 < n; k0 += kChunkWide * kW)
      merge_chunk<kChunkWide>(a.ws_o + base * kDV + lane * 8, a.ws_lse + base, stride, k0, n, st);
  }
  acc_s[w][0][lane] = st.acc0;
  acc_s[w][1][lane] = st.acc1;
  if (lane == 0) {
    ml_s[w][0] = st.m;
    ml_s[w][1] = st.l;
  }
  __syncthreads();
  if (w != 0) return;
  MergeState t{-INFINITY, 0.f, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int u = 0; u < kW; ++u) t.m = fmaxf(t.m, ml_s[u][0]);
  if (t.m != -INFINITY) {
#pragma unroll
    for (int u = 0; u < kW; ++u) {
      const float mu = ml_s[u][0];
      if (mu == -INFINITY) continue;   // a wave whose splits saw no key (uniform)
      const float c = __builtin_amdgcn_exp2f((mu - t.m) * kLog2e);
      t.l += c * ml_s[u][1];
      t.acc0 += c * acc_s[u][0][lane];
      t.acc1 += c * acc_s[u][1][lane];
    }
  }
  store_merged(a, (int64_t)(q0 + i) * a.heads + h, lane, t);
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

hipError_t launch_merge(const MergeArgs& a, int rows, int heads, int q_len_max, int max_splits, hipStream_t st) {
  void* args[] = {(void*)&a};
  constexpr int kW = kBlockThreads / 64;
  if (max_splits > kChunkWide)   // some row needs more than one round trip per wave
    return hipLaunchKernel((const void*)merge_wide_kernel, dim3(rows * q_len_max * heads), dim3(kWideThreads), args,
                           0, st);
  dim3 grid(rows * q_len_max * ((heads + kW - 1) / kW));
  const void* fn = max_splits <= 2   ? (const void*)merge_kernel<2>
                   : max_splits <= 4 ? (const void*)merge_kernel<4>
                                     : (const void*)merge_kernel<8>;
  return hipLaunchKernel(fn, grid, dim3(kBlockThreads), args, 0, st);
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
