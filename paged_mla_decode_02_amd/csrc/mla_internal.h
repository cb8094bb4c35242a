// Internal declarations shared by the library's host sources (not installed).
#pragma once

#include <cstdint>
#include <string>

#include "mla_decode.h"

namespace mla {

// Plan spec version 4 constants. The decode kernel's tile is compiled for
// kMUnit query rows; the planner writes the same value into every plan header
// and the launcher refuses a plan whose header differs.
constexpr int32_t kPlanMagic = 0x4D4C4150;
constexpr int32_t kPlanVersion = 4;
constexpr int32_t kHeaderWords = 20;
constexpr int32_t kMUnit = 128;
constexpr int32_t kNMax = 256;
constexpr int32_t kMinSplitKeys = 256;
constexpr int32_t kItemOverhead = 256;
constexpr int32_t kOcc = 1;
constexpr int32_t kXcds = 8;

// Workspace layout: the bf16 partial O and fp32 LSE of the split rows; with an
// in-kernel-merge plan, a fixed region of split-arrival counters (one per
// request row and M tile, zero between calls) comes first. With such a plan,
// rows with at most kMaxInKernelSplits splits are merged inside the decode
// kernel by the last of their splits to finish; rows with more (and every
// split row when rows * u exceeds the counters) go to the merge kernel.
constexpr int64_t kWsCounterBytes = 256 * 1024;
constexpr int32_t kWsCounters = (int32_t)(kWsCounterBytes / 4);
constexpr int32_t kMaxInKernelSplits = 16;

enum HeaderField : int {
  H_MAGIC = 0, H_VERSION, H_ROWS, H_HEADS, H_QLEN, H_KVDTYPE, H_CUS, H_MODE, H_MUNIT, H_U,
  H_NMAX, H_MINSPLIT, H_OVERHEAD, H_OCC, H_S, H_W, H_G, H_P, H_HWORDS, H_TOTAL
};

// Offsets (in words) of the plan's arrays, from its header.
struct PlanView {
  int32_t rows, heads, q_len_max, kv_dtype, mode, m_unit, u, S, W, G, P, total;
  int32_t max_splits;   // largest split count of a row
  bool merge_in_kernel; // the caller asked for the split merge inside the decode kernel
  bool pv_fp8;          // the caller asked for fp8 PV products (fp8 KV)
  int64_t off_split_indptr, off_split_row, off_split_begin, off_split_end, off_split_part,
      off_work_indptr, off_item_split, off_item_m;
};

// Parses and checks a plan header; returns MLA_OK or an error (message set).
int32_t view_plan(const int32_t* plan, PlanView* v);

// Workspace bytes a plan needs (0 when no row is split).
inline int64_t workspace_counter_bytes(const PlanView& v) { return v.merge_in_kernel ? kWsCounterBytes : 0; }
inline int64_t workspace_bytes(const PlanView& v) {
  if (v.P == 0) return 0;
  // bf16 partial O, then fp32 partial LSE
  return workspace_counter_bytes(v) + (int64_t)v.P * v.q_len_max * v.heads * (MLA_D_V * 2 + 4);
}

int32_t set_error(int32_t status, const std::string& msg);
void clear_error();

// The checks and launches behind mla_decode_fwd (dcp_world 1, dcp_rank 0,
// kv_len_global null), mla_decode_fwd_dcp and mla_decode_fwd_noalloc. With
// clear_counters, an in-kernel-merge plan's split-arrival counters are zeroed
// by a fill kernel right before the decode (after every check has passed).
int32_t decode_impl(const void* q, mla_dtype q_dtype, const float* q_scale, const void* kv_pool,
                    mla_dtype kv_dtype, const float* kv_scale, int64_t num_slots,
                    const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                    const int32_t* plan_host, const int32_t* plan_dev, int32_t rows,
                    int32_t num_heads, int32_t q_len_max, int32_t causal, float softmax_scale,
                    void* o, float* lse, void* workspace, int64_t workspace_bytes, void* stream,
                    int32_t dcp_world, int32_t dcp_rank, const int32_t* kv_len_global,
                    bool clear_counters = false);

}  // namespace mla
