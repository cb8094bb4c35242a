// Host split planner (plan spec version 4).
//
// A plan is a split count and split_indptr per request row, built on the host
// next to the decode CSR ([DSV4] Tuned ASM FP8 decode with split plans, ATOM
// pull request 2462, Summary part 1). UNIFORM plans depend only on the row
// count, the longest row and the config (the same page: such plans keep graph
// capture and replay in agreement); LENGTH_AWARE plans follow the real per-row
// lengths on every call, as the persistent decode kernel of the same page does
// (Summary part 2). AUTO builds both and keeps the one with the shorter
// estimated duration.
//
// On top of the splits the plan fixes the launch. Work items are (split,
// tile of 128 query rows); all M tiles of one split read the same keys, so
// they run on one chiplet (XCD) and share its L2. UNIFORM ranks splits
// longest first, deals them to the eight chiplets and launches one workgroup
// per item, ordering workgroup ids so that the hardware's round-robin
// dispatch over chiplets lands each chiplet's items on it. LENGTH_AWARE packs
// the rows, longest first, into lanes of equal capacity -- a lane being u
// workgroups of one chiplet that run the same splits, one M tile each --
// cutting a row only where a lane is full, and launches those workgroups
// persistently.
#include <algorithm>
#include <cstring>
#include <numeric>
#include <vector>

#include "mla_internal.h"

namespace mla {
namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Item {
  int32_t split, m;
};

}  // namespace

int32_t view_plan(const int32_t* plan, PlanView* v) {
  if (!plan) return set_error(MLA_ERR_INVALID_ARG, "plan is null");
  if (plan[H_MAGIC] != kPlanMagic) return set_error(MLA_ERR_PLAN_MISMATCH, "plan magic mismatch");
  if (plan[H_VERSION] != kPlanVersion || plan[H_HWORDS] != kHeaderWords)
    return set_error(MLA_ERR_PLAN_MISMATCH, "plan from a different spec version");
  v->rows = plan[H_ROWS];
  v->heads = plan[H_HEADS];
  v->q_len_max = plan[H_QLEN];
  v->kv_dtype = plan[H_KVDTYPE];
  v->mode = plan[H_MODE] & ~(MLA_PLAN_MERGE_IN_KERNEL | MLA_PLAN_FP8_PV);
  v->merge_in_kernel = (plan[H_MODE] & MLA_PLAN_MERGE_IN_KERNEL) != 0;
  v->pv_fp8 = (plan[H_MODE] & MLA_PLAN_FP8_PV) != 0;
  v->m_unit = plan[H_MUNIT];
  v->u = plan[H_U];
  v->S = plan[H_S];
  v->W = plan[H_W];
  v->G = plan[H_G];
  v->P = plan[H_P];
  v->total = plan[H_TOTAL];
  if (v->rows < 1 || v->S < v->rows || v->W != (int64_t)v->S * v->u || v->G < 1 || v->P < 0 ||
      v->P > v->S || v->m_unit != kMUnit ||
      (v->pv_fp8 && (v->kv_dtype != MLA_FP8_E4M3 || v->merge_in_kernel)))
    return set_error(MLA_ERR_PLAN_MISMATCH, "plan header is inconsistent");
  int64_t off = kHeaderWords;
  v->off_split_indptr = off; off += v->rows + 1;
  v->off_split_row = off; off += v->S;
  v->off_split_begin = off; off += v->S;
  v->off_split_end = off; off += v->S;
  v->off_split_part = off; off += v->S;
  v->off_work_indptr = off; off += v->G + 1;
  v->off_item_split = off; off += v->W;
  v->off_item_m = off; off += v->W;
  if (off != v->total) return set_error(MLA_ERR_PLAN_MISMATCH, "plan length mismatch");
  // The merge kernel takes up to four splits per lane of a wave: at most
  // N_MAX = 256 splits per row, and split_indptr must run from 0 to S.
  if (plan[H_NMAX] != kNMax || plan[v->off_split_indptr] != 0 ||
      plan[v->off_split_indptr + v->rows] != v->S)
    return set_error(MLA_ERR_PLAN_MISMATCH, "plan split_indptr is inconsistent");
  v->max_splits = 0;
  for (int32_t b = 0; b < v->rows; ++b) {
    const int32_t n = plan[v->off_split_indptr + b + 1] - plan[v->off_split_indptr + b];
    if (n < 1 || n > kNMax)
      return set_error(MLA_ERR_PLAN_MISMATCH, "plan has a row with no split or more than 256");
    v->max_splits = n > v->max_splits ? n : v->max_splits;
  }
  return MLA_OK;
}

}  // namespace mla

using namespace mla;

extern "C" int32_t mla_decode_plan_capacity(int32_t rows, int32_t num_cus, int32_t num_heads,
                                            int32_t q_len_max, int64_t* words_out) {
  clear_error();
  if (!words_out) return set_error(MLA_ERR_INVALID_ARG, "words_out is null");
  if (rows < 1 || num_cus < 1) return set_error(MLA_ERR_INVALID_ARG, "rows and num_cus must be >= 1");
  if (num_heads < 1 || num_heads > MLA_MAX_HEADS || q_len_max < 1 || q_len_max > MLA_MAX_Q_LEN)
    return set_error(MLA_ERR_UNSUPPORTED, "heads must be 1..128 and q_len_max 1..16");
  const int64_t u = cdiv((int64_t)num_heads * q_len_max, kMUnit);
  // UNIFORM: S <= rows * N_MAX and G = W; LENGTH_AWARE: S <= rows + lanes - 1
  // <= rows + OCC * CUs and G <= max(OCC * CUs, u).
  const int64_t s_max = std::max<int64_t>((int64_t)rows * kNMax, (int64_t)rows + (int64_t)kOcc * num_cus);
  const int64_t w_max = s_max * u;
  const int64_t g_max = std::max<int64_t>(w_max, std::max<int64_t>((int64_t)kOcc * num_cus, u));
  *words_out = kHeaderWords + (rows + 1) + 4 * s_max + (g_max + 1) + 2 * w_max;
  return MLA_OK;
}

extern "C" int32_t mla_decode_plan(const int32_t* kv_lens, int32_t rows, int32_t num_heads,
                                   int32_t q_len_max, mla_dtype kv_dtype, mla_plan_mode mode,
                                   int32_t num_cus, int32_t* plan, int64_t plan_words) {
  clear_error();
  if (!kv_lens || !plan) return set_error(MLA_ERR_INVALID_ARG, "kv_lens and plan must be non-null");
  if (rows < 1 || rows > (1 << 24)) return set_error(MLA_ERR_UNSUPPORTED, "rows must be in 1..2^24");
  if (num_heads < 1 || num_heads > MLA_MAX_HEADS)
    return set_error(MLA_ERR_UNSUPPORTED, "num_heads must be in 1..128");
  if (q_len_max < 1 || q_len_max > MLA_MAX_Q_LEN)
    return set_error(MLA_ERR_UNSUPPORTED, "q_len_max must be in 1..16");
  if (kv_dtype != MLA_BF16 && kv_dtype != MLA_FP8_E4M3)
    return set_error(MLA_ERR_INVALID_ARG, "unknown kv_dtype");
  const int32_t flag = (int32_t)mode & (MLA_PLAN_MERGE_IN_KERNEL | MLA_PLAN_FP8_PV);
  const int32_t base_mode = (int32_t)mode & ~(MLA_PLAN_MERGE_IN_KERNEL | MLA_PLAN_FP8_PV);
  if (base_mode != MLA_PLAN_AUTO && base_mode != MLA_PLAN_UNIFORM && base_mode != MLA_PLAN_LENGTH_AWARE)
    return set_error(MLA_ERR_INVALID_ARG, "unknown plan mode");
  if ((flag & MLA_PLAN_FP8_PV) && kv_dtype != MLA_FP8_E4M3)
    return set_error(MLA_ERR_UNSUPPORTED, "MLA_PLAN_FP8_PV needs fp8 KV");
  if ((flag & MLA_PLAN_FP8_PV) && (flag & MLA_PLAN_MERGE_IN_KERNEL))
    return set_error(MLA_ERR_UNSUPPORTED, "MLA_PLAN_FP8_PV does not combine with MLA_PLAN_MERGE_IN_KERNEL");
  if (num_cus < 1) return set_error(MLA_ERR_INVALID_ARG, "num_cus must be >= 1");

  int64_t sum_len = 0, max_len = 0;
  for (int32_t b = 0; b < rows; ++b) {
    if (kv_lens[b] < 0) return set_error(MLA_ERR_INVALID_ARG, "negative KV length");
    sum_len += kv_lens[b];
    max_len = std::max<int64_t>(max_len, kv_lens[b]);
  }
  if (sum_len > INT32_MAX) return set_error(MLA_ERR_UNSUPPORTED, "total KV length exceeds int32");

  const int64_t u = cdiv((int64_t)num_heads * q_len_max, kMUnit);

  // Splits of each mode: (row, key range), in row order.
  struct Splits {
    std::vector<int32_t> row, beg, end;
  };
  Splits uni, la;
  std::vector<int32_t> la_lane;   // LENGTH_AWARE: each split's lane
  int32_t X = kXcds;
  int64_t n_lanes = 0, la_est = 0;
  if (base_mode != MLA_PLAN_LENGTH_AWARE) {
    int64_t n = std::min(cdiv((int64_t)kOcc * num_cus, (int64_t)rows * u), cdiv(max_len, kMinSplitKeys));
    n = std::clamp<int64_t>(n, 1, kNMax);
    if ((int64_t)rows * n > INT32_MAX) return set_error(MLA_ERR_UNSUPPORTED, "too many splits");
    uni.row.reserve(rows * n);
    for (int32_t b = 0; b < rows; ++b)
      for (int64_t k = 0; k < n; ++k) {
        uni.row.push_back(b);
        uni.beg.push_back((int32_t)(k * kv_lens[b] / n));
        uni.end.push_back((int32_t)((k + 1) * kv_lens[b] / n));
      }
  }
  if (base_mode != MLA_PLAN_UNIFORM) {
    // Lanes: u workgroups of one chiplet that run the same splits, one M
    // tile each, all with room T (keys + kItemOverhead per split). Rows go
    // longest first (ties by index) to the roomiest lane (lowest index among
    // equals); a row is cut only where that lane is full.
    const int64_t slots = (int64_t)kOcc * num_cus;
    while (X > 1 && slots / X < u) X /= 2;
    const int64_t lam = std::max<int64_t>(1, (slots / X) / u);
    n_lanes = X * lam;
    const int64_t T = std::max({(int64_t)kMinSplitKeys + kItemOverhead,
                                cdiv(sum_len + (int64_t)kItemOverhead * (rows + n_lanes), n_lanes),
                                cdiv(max_len, kNMax - 1) + kItemOverhead});
    std::vector<int64_t> room(n_lanes, T);
    auto roomiest = [&]() {
      int64_t best = 0;
      for (int64_t l = 1; l < n_lanes; ++l)
        if (room[l] > room[best]) best = l;
      return best;
    };
    std::vector<int32_t> order(rows);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return kv_lens[a] > kv_lens[b]; });
    struct Piece {
      int32_t row, begin, end, lane;
    };
    std::vector<Piece> pieces;
    pieces.reserve(rows + n_lanes);
    for (int32_t b : order) {
      const int64_t L = kv_lens[b];
      if (L == 0) {
        pieces.push_back({b, 0, 0, (int32_t)roomiest()});
        continue;
      }
      int32_t count = 0;
      for (int64_t pos = 0; pos < L; ++count) {
        const int64_t lane = roomiest();
        const int64_t r = room[lane] - kItemOverhead;
        const int64_t take = (r >= L - pos || r < kMinSplitKeys || count == kNMax - 1) ? L - pos : r;
        pieces.push_back({b, (int32_t)pos, (int32_t)(pos + take), (int32_t)lane});
        room[lane] -= take + kItemOverhead;
        pos += take;
      }
    }
    // Split ids in (row, first key) order.
    std::sort(pieces.begin(), pieces.end(),
              [](const Piece& a, const Piece& b) { return a.row != b.row ? a.row < b.row : a.begin < b.begin; });
    for (const Piece& p : pieces) {
      la.row.push_back(p.row);
      la.beg.push_back(p.begin);
      la.end.push_back(p.end);
      la_lane.push_back(p.lane);
    }
    la_est = T - *std::min_element(room.begin(), room.end());   // the fullest lane's cost
  }

  // AUTO: the mode whose duration estimate (keys, kItemOverhead per split) is
  // smaller; UNIFORM's is max(costliest split, cdiv(u * total cost, OCC *
  // CUs)), LENGTH_AWARE's its fullest lane; ties go to UNIFORM.
  int32_t used = base_mode;
  if (used == MLA_PLAN_AUTO) {
    int64_t max_cost = 0, sum_cost = 0;
    for (size_t s = 0; s < uni.row.size(); ++s) {
      const int64_t c = (int64_t)uni.end[s] - uni.beg[s] + kItemOverhead;
      max_cost = std::max(max_cost, c);
      sum_cost += c;
    }
    const int64_t uni_est = std::max(max_cost, cdiv(u * sum_cost, (int64_t)kOcc * num_cus));
    used = la_est < uni_est ? MLA_PLAN_LENGTH_AWARE : MLA_PLAN_UNIFORM;
  }
  const Splits& sp = used == MLA_PLAN_UNIFORM ? uni : la;
  const std::vector<int32_t>& srow = sp.row;
  const std::vector<int32_t>& sbeg = sp.beg;
  const std::vector<int32_t>& send = sp.end;
  std::vector<std::vector<int32_t>> lane_splits;   // LENGTH_AWARE: each lane's splits by id
  if (used == MLA_PLAN_LENGTH_AWARE) {
    lane_splits.resize(n_lanes);
    for (size_t s = 0; s < la_lane.size(); ++s) lane_splits[la_lane[s]].push_back((int32_t)s);
  }
  const int32_t S = (int32_t)srow.size();

  // Split CSR and partial slots.
  std::vector<int32_t> split_indptr(rows + 1, 0);
  for (int32_t s = 0; s < S; ++s) ++split_indptr[srow[s] + 1];
  for (int32_t b = 0; b < rows; ++b) split_indptr[b + 1] += split_indptr[b];
  std::vector<int32_t> spart(S);
  int32_t P = 0;
  for (int32_t s = 0; s < S; ++s)
    spart[s] = split_indptr[srow[s] + 1] - split_indptr[srow[s]] > 1 ? P++ : -1;

  const int64_t W64 = (int64_t)S * u;
  if (W64 > INT32_MAX) return set_error(MLA_ERR_UNSUPPORTED, "too many work items");
  const int32_t W = (int32_t)W64;

  // Workgroups.
  int32_t G = 0;
  std::vector<int32_t> work_indptr;
  std::vector<Item> items;
  items.reserve(W);
  if (used == MLA_PLAN_UNIFORM) {
    // Rank splits longest first and deal them to chiplets; workgroup ids are
    // ordered so that the hardware's round-robin dispatch over chiplets lands
    // each chiplet's items on it.
    G = W;
    std::vector<int64_t> cost(S);
    for (int32_t s = 0; s < S; ++s) cost[s] = (int64_t)send[s] - sbeg[s] + kItemOverhead;
    std::vector<int32_t> rank(S);
    std::iota(rank.begin(), rank.end(), 0);
    std::stable_sort(rank.begin(), rank.end(), [&](int32_t a, int32_t b) { return cost[a] > cost[b]; });
    std::vector<std::vector<Item>> chiplet(kXcds);
    for (int32_t k = 0; k < S; ++k)
      for (int32_t m = 0; m < (int32_t)u; ++m) chiplet[k % kXcds].push_back({rank[k], m});
    std::vector<Item> by_id(W);
    size_t n_min = SIZE_MAX, n_max = 0;
    for (auto& c : chiplet) { n_min = std::min(n_min, c.size()); n_max = std::max(n_max, c.size()); }
    for (int32_t x = 0; x < kXcds; ++x)
      for (size_t j = 0; j < n_min; ++j) by_id[(size_t)kXcds * j + x] = chiplet[x][j];
    size_t next = (size_t)kXcds * n_min;
    for (size_t j = n_min; j < n_max; ++j)
      for (int32_t x = 0; x < kXcds; ++x)
        if (j < chiplet[x].size()) by_id[next++] = chiplet[x][j];
    items = by_id;
    work_indptr.resize(G + 1);
    for (int32_t g = 0; g <= G; ++g) work_indptr[g] = g;
  } else {
    // Member j of lane l (chiplet x = l mod X, k = l / X) is workgroup
    // x + X (k u + j) and runs (s, j) for the lane's splits s in order.
    std::vector<int32_t> lane_of_wg, member_of_wg;
    for (int64_t l = 0; l < (int64_t)lane_splits.size(); ++l) {
      if (lane_splits[l].empty()) continue;
      const int64_t x = l % X, k = l / X;
      for (int64_t j = 0; j < u; ++j) {
        const int64_t g = x + X * (k * u + j);
        if (g >= (int64_t)lane_of_wg.size()) {
          lane_of_wg.resize(g + 1, -1);
          member_of_wg.resize(g + 1, -1);
        }
        lane_of_wg[g] = (int32_t)l;
        member_of_wg[g] = (int32_t)j;
      }
    }
    G = (int32_t)lane_of_wg.size();
    work_indptr.assign(G + 1, 0);
    for (int32_t g = 0; g < G; ++g) {
      if (lane_of_wg[g] >= 0)
        for (int32_t s : lane_splits[lane_of_wg[g]]) items.push_back({s, member_of_wg[g]});
      work_indptr[g + 1] = (int32_t)items.size();
    }
  }

  const int64_t total = kHeaderWords + (rows + 1) + 4 * (int64_t)S + (G + 1) + 2 * (int64_t)W;
  if (total > plan_words) return set_error(MLA_ERR_INVALID_ARG, "plan buffer too small");
  int32_t* w = plan;
  const int32_t header[kHeaderWords] = {kPlanMagic, kPlanVersion, rows, num_heads, q_len_max,
                                        (int32_t)kv_dtype, num_cus, used | flag, kMUnit, (int32_t)u,
                                        kNMax, kMinSplitKeys, kItemOverhead, kOcc, S, W, G, P,
                                        kHeaderWords, (int32_t)total};
  std::memcpy(w, header, sizeof(header));
  w += kHeaderWords;
  auto put = [&](const std::vector<int32_t>& a) { std::memcpy(w, a.data(), a.size() * 4); w += a.size(); };
  put(split_indptr);
  put(srow);
  put(sbeg);
  put(send);
  put(spart);
  put(work_indptr);
  for (const Item& it : items) *w++ = it.split;
  for (const Item& it : items) *w++ = it.m;
  return MLA_OK;
}

extern "C" int32_t mla_decode_workspace_size(const int32_t* plan, int64_t* bytes_out) {
  clear_error();
  if (!bytes_out) return set_error(MLA_ERR_INVALID_ARG, "bytes_out is null");
  PlanView v;
  int32_t st = view_plan(plan, &v);
  if (st != MLA_OK) return st;
  *bytes_out = workspace_bytes(v);
  return MLA_OK;
}
