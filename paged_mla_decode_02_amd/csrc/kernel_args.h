// Kernel argument blocks and launchers (internal; shared by api.cpp and
// kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mla {

// Everything the decode kernel reads, by value. Plan arrays are addressed as
// plan + off_*, offsets taken from the host copy of the plan header.
struct DecodeArgs {
  const void* q;
  const float* q_scale;     // device scalar or null
  const void* kv;
  const float* kv_scale;    // device scalar or null
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* plan;
  int32_t off_split_row, off_split_begin, off_split_end, off_split_part;
  int32_t off_work_indptr, off_item_split, off_item_m;
  int32_t heads, q_len_max, causal;
  uint32_t max_slot;         // num_slots - 1: slot lists are clamped to the pool
  float score_scale_log2;   // softmax_scale * log2(e)
  int32_t dcp_world, dcp_rank;      // round-robin KV shard: local key j at position j * world + rank
  int32_t* counters;        // [rows * u] split arrivals per (row, M tile); zero between calls
  int32_t off_split_indptr, u;
  int32_t inkernel_max_splits;   // rows with 1 < n <= this many splits merge in the decode kernel
  int32_t uniform_ranges;   // split k of n covers [k L / n, (k + 1) L / n) of the live length L
  const int32_t* kv_len_global;     // [rows] keys of each row over all shards, or null (= local)
  uint16_t* o;              // bf16 bits
  float* lse;
  uint16_t* ws_o;           // [P, q_len_max, heads, 512] bf16 partial O (normalized)
  float* ws_lse;            // [P, q_len_max, heads] fp32 partial LSE
};

struct MergeArgs {
  const int32_t* qo_indptr;
  const int32_t* plan;
  int32_t off_split_indptr, off_split_part;
  int32_t heads, q_len_max;
  const uint16_t* ws_o;
  const float* ws_lse;
  uint16_t* o;
  float* lse;
  int32_t skip_upto;        // rows with at most this many splits were merged in the decode kernel
};

struct GatherArgs {
  const void* kv;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* plan;
  int32_t off_split_row, off_split_begin, off_split_end, off_split_indptr;
  int32_t uniform_ranges;
  uint32_t max_slot;         // num_slots - 1
  uint16_t* dense;          // bf16 [nnz, 576]
};

struct ShardMergeArgs {
  const uint16_t* o_parts;  // bf16 [world, rows, 512]
  const float* lse_parts;   // [world, rows]
  int32_t world, rows;      // rows = tokens * heads
  uint16_t* o;              // bf16 [rows, 512]
  float* lse;               // [rows]
};

struct CacheWriteArgs {
  const void* kv_c;         // [tokens] rows of 512 at kv_c_stride elements
  const void* k_pe;         // [tokens] rows of 64 at k_pe_stride elements
  int32_t kv_c_dtype, k_pe_dtype;   // mla_src_dtype
  int64_t kv_c_stride, k_pe_stride;
  const int64_t* slots;     // [tokens]
  int32_t tokens, kv_fp8;
  void* pool;               // [num_slots, 576]
  const float* kv_scale;    // device scalar or null
  int64_t num_slots;
};

constexpr int kBlockThreads = 256;   // merge kernel: 4 waves of 64, one block per (row, token, head)
constexpr int kDecodeThreads = 256;  // decode and gather kernels: 4 waves of 64, one per SIMD

// pv_fp8: the fp8 PV products (fp8 KV only).
hipError_t launch_decode(const DecodeArgs& a, bool q_fp8, bool kv_fp8, bool pv_fp8, int grid, hipStream_t st);
// max_splits: the plan's largest split count of a row (picks the merge layout).
hipError_t launch_merge(const MergeArgs& a, int rows, int heads, int q_len_max, int max_splits, hipStream_t st);
hipError_t launch_gather(const GatherArgs& a, bool kv_fp8, int splits, hipStream_t st);
hipError_t launch_shard_merge(const ShardMergeArgs& a, hipStream_t st);
hipError_t launch_zero(uint32_t* p, int32_t words, hipStream_t st);
// vec: every source row and the pool are 16-byte aligned (8-element chunks).
hipError_t launch_cache_write(const CacheWriteArgs& a, bool vec, hipStream_t st);

}  // namespace mla
