// Internal declarations shared by the library's host sources (not installed).
#pragma once

#include <cstdint>
#include <string>

#include "mla_decode.h"

namespace mla {

// Plan spec version 1 constants. The decode kernel's tile is compiled for
// kMUnit query rows; the planner writes the same value into every plan header
// and the launcher refuses a plan whose header differs.
constexpr int32_t kPlanMagic = 0x4D4C4150;
constexpr int32_t kPlanVersion = 1;
constexpr int32_t kHeaderWords = 20;
constexpr int32_t kMUnit = 64;
constexpr int32_t kNMax = 64;
constexpr int32_t kMinSplitKeys = 256;
constexpr int32_t kItemOverhead = 64;
constexpr int32_t kOcc = 2;
constexpr int32_t kXcds = 8;

enum HeaderField : int {
  H_MAGIC = 0, H_VERSION, H_ROWS, H_HEADS, H_QLEN, H_KVDTYPE, H_CUS, H_MODE, H_MUNIT, H_U,
  H_NMAX, H_MINSPLIT, H_OVERHEAD, H_OCC, H_S, H_W, H_G, H_P, H_HWORDS, H_TOTAL
};

// Offsets (in words) of the plan's arrays, from its header.
struct PlanView {
  int32_t rows, heads, q_len_max, kv_dtype, mode, m_unit, u, S, W, G, P, total;
  int64_t off_split_indptr, off_split_row, off_split_begin, off_split_end, off_split_part,
      off_work_indptr, off_item_split, off_item_m;
};

// Parses and checks a plan header; returns MLA_OK or an error (message set).
int32_t view_plan(const int32_t* plan, PlanView* v);

int32_t set_error(int32_t status, const std::string& msg);
void clear_error();

}  // namespace mla
