// C ABI entry points: host-side validation, then the launches.
//
// Everything the library can check without touching device memory is checked
// here, before any launch, and reported as a status code; a missing kernel or
// an unsupported shape is never a process abort (the failure mode the
// non-causal draft page reports for a kernel lookup miss, vLLM pull request
// 53001, Purpose). A dtype mismatch is refused, never reinterpreted (the
// review thread of vLLM pull request 57942 traces corrupted cache rows to an
// fp32 tensor read as bf16).
#include <cmath>
#include <cstdint>
#include <string>

#include "kernel_args.h"
#include "mla_internal.h"

using namespace mla;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_dtype(int d) { return d == MLA_BF16 || d == MLA_FP8_E4M3; }

int32_t check_plan_for_call(const int32_t* plan_host, const int32_t* plan_dev, int32_t rows,
                            int32_t heads, int32_t q_len_max, int32_t kv_dtype, PlanView* v) {
  if (!plan_dev) return set_error(MLA_ERR_INVALID_ARG, "plan_dev is null");
  int32_t st = view_plan(plan_host, v);
  if (st != MLA_OK) return st;
  if (v->rows != rows) return set_error(MLA_ERR_PLAN_MISMATCH, "plan was built for a different row count");
  if (v->heads != heads) return set_error(MLA_ERR_PLAN_MISMATCH, "plan was built for a different head count");
  if (v->q_len_max != q_len_max)
    return set_error(MLA_ERR_PLAN_MISMATCH, "plan was built for a different q_len_max");
  if (v->kv_dtype != kv_dtype) return set_error(MLA_ERR_PLAN_MISMATCH, "plan was built for a different KV dtype");
  return MLA_OK;
}

}  // namespace

// Shared by mla_decode_fwd (world 1), mla_decode_fwd_dcp and
// mla_decode_fwd_noalloc.
int32_t mla::decode_impl(const void* q, mla_dtype q_dtype, const float* q_scale, const void* kv_pool,
                    mla_dtype kv_dtype, const float* kv_scale, int64_t num_slots,
                    const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                    const int32_t* plan_host, const int32_t* plan_dev, int32_t rows,
                    int32_t num_heads, int32_t q_len_max, int32_t causal, float softmax_scale,
                    void* o, float* lse, void* workspace, int64_t workspace_bytes, void* stream,
                    int32_t dcp_world, int32_t dcp_rank, const int32_t* kv_len_global,
                    bool clear_counters) {
  if (!q || !kv_pool || !qo_indptr || !kv_indptr || !kv_indices || !plan_host || !o || !lse)
    return set_error(MLA_ERR_INVALID_ARG, "a required pointer is null");
  if (!valid_dtype(q_dtype) || !valid_dtype(kv_dtype))
    return set_error(MLA_ERR_INVALID_ARG, "unknown dtype (expected MLA_BF16 or MLA_FP8_E4M3)");
  if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(o))
    return set_error(MLA_ERR_INVALID_ARG, "q, kv_pool and o must be 16-byte aligned");
  if (rows < 1) return set_error(MLA_ERR_INVALID_ARG, "rows must be >= 1");
  if (num_heads < 1 || num_heads > MLA_MAX_HEADS)
    return set_error(MLA_ERR_UNSUPPORTED, "num_heads must be in 1..128");
  if (q_len_max < 1 || q_len_max > MLA_MAX_Q_LEN)
    return set_error(MLA_ERR_UNSUPPORTED, "q_len_max must be in 1..16");
  if (causal != 0 && causal != 1) return set_error(MLA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return set_error(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (num_slots < 1 || num_slots > ((int64_t)1 << 31))
    return set_error(MLA_ERR_INVALID_ARG, "num_slots must be in 1..2^31");
  PlanView v;
  int32_t st = check_plan_for_call(plan_host, plan_dev, rows, num_heads, q_len_max, kv_dtype, &v);
  if (st != MLA_OK) return st;
  const int64_t need = mla::workspace_bytes(v);
  if (need > 0) {
    if (!workspace) return set_error(MLA_ERR_WORKSPACE, "this plan needs a workspace");
    if (workspace_bytes < need)
      return set_error(MLA_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
    if (!aligned16(workspace)) return set_error(MLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  const int64_t max_tokens = (int64_t)rows * q_len_max;
  if (max_tokens * num_heads * MLA_D_LATENT > ((int64_t)1 << 40))
    return set_error(MLA_ERR_UNSUPPORTED, "query tensor too large");

  DecodeArgs a;
  a.q = q;
  a.q_scale = q_scale;
  a.kv = kv_pool;
  a.kv_scale = kv_scale;
  a.max_slot = (uint32_t)(num_slots - 1);
  a.qo_indptr = qo_indptr;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.plan = plan_dev;
  a.off_split_row = (int32_t)v.off_split_row;
  a.off_split_begin = (int32_t)v.off_split_begin;
  a.off_split_end = (int32_t)v.off_split_end;
  a.off_split_part = (int32_t)v.off_split_part;
  a.off_work_indptr = (int32_t)v.off_work_indptr;
  a.off_item_split = (int32_t)v.off_item_split;
  a.off_item_m = (int32_t)v.off_item_m;
  a.heads = num_heads;
  a.q_len_max = q_len_max;
  a.causal = causal;
  a.score_scale_log2 = softmax_scale * 1.44269504088896340736f;
  a.dcp_world = dcp_world;
  a.dcp_rank = dcp_rank;
  a.kv_len_global = kv_len_global;
  a.o = (uint16_t*)o;
  a.lse = lse;
  const int64_t ws_o_elems = (int64_t)v.P * q_len_max * num_heads * MLA_D_V;
  uint16_t* partials = need > 0 ? (uint16_t*)((char*)workspace + workspace_counter_bytes(v)) : nullptr;
  a.ws_o = partials;
  a.ws_lse = need > 0 ? (float*)(partials + ws_o_elems) : nullptr;
  a.counters = need > 0 ? (int32_t*)workspace : nullptr;
  a.off_split_indptr = (int32_t)v.off_split_indptr;
  a.u = v.u;
  // split rows with up to kMaxInKernelSplits splits merge inside the decode
  // kernel when every (row, M tile) has a counter
  a.inkernel_max_splits =
      (need > 0 && v.merge_in_kernel && (int64_t)rows * v.u <= kWsCounters) ? kMaxInKernelSplits : 1;
  // a UNIFORM plan's split ranges follow from the live lengths (k L / n), so
  // such a plan stays valid when the lengths change (graph replay)
  a.uniform_ranges = v.mode == MLA_PLAN_UNIFORM;

  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (clear_counters && a.inkernel_max_splits > 1) {
    e = launch_zero((uint32_t*)a.counters, rows * v.u, s);
    if (e != hipSuccess) return set_error(MLA_ERR_HIP, std::string("counter clear launch: ") + hipGetErrorString(e));
  }
  e = launch_decode(a, q_dtype == MLA_FP8_E4M3, kv_dtype == MLA_FP8_E4M3, v.pv_fp8, v.G, s);
  if (e != hipSuccess) return set_error(MLA_ERR_HIP, std::string("decode launch: ") + hipGetErrorString(e));
  if (v.P > 0 && v.max_splits > a.inkernel_max_splits) {
    MergeArgs mg;
    mg.qo_indptr = qo_indptr;
    mg.plan = plan_dev;
    mg.off_split_indptr = (int32_t)v.off_split_indptr;
    mg.off_split_part = (int32_t)v.off_split_part;
    mg.heads = num_heads;
    mg.q_len_max = q_len_max;
    mg.ws_o = a.ws_o;
    mg.ws_lse = a.ws_lse;
    mg.skip_upto = a.inkernel_max_splits;
    mg.o = a.o;
    mg.lse = lse;
    e = launch_merge(mg, rows, num_heads, q_len_max, v.max_splits, s);
    if (e != hipSuccess) return set_error(MLA_ERR_HIP, std::string("merge launch: ") + hipGetErrorString(e));
  }
  return MLA_OK;
}

extern "C" int32_t mla_decode_fwd(const void* q, mla_dtype q_dtype, const float* q_scale,
                                  const void* kv_pool, mla_dtype kv_dtype, const float* kv_scale,
                                  int64_t num_slots, const int32_t* qo_indptr,
                                  const int32_t* kv_indptr, const int32_t* kv_indices,
                                  const int32_t* plan_host, const int32_t* plan_dev, int32_t rows,
                                  int32_t num_heads, int32_t q_len_max, int32_t causal,
                                  float softmax_scale, void* o, float* lse, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
  clear_error();
  return decode_impl(q, q_dtype, q_scale, kv_pool, kv_dtype, kv_scale, num_slots, qo_indptr,
                     kv_indptr, kv_indices, plan_host, plan_dev, rows, num_heads, q_len_max, causal,
                     softmax_scale, o, lse, workspace, workspace_bytes, stream, 1, 0, nullptr);
}

extern "C" int32_t mla_decode_fwd_dcp(const void* q, mla_dtype q_dtype, const float* q_scale,
                                      const void* kv_pool, mla_dtype kv_dtype, const float* kv_scale,
                                      int64_t num_slots, const int32_t* qo_indptr,
                                      const int32_t* kv_indptr, const int32_t* kv_indices,
                                      const int32_t* plan_host, const int32_t* plan_dev,
                                      int32_t rows, int32_t num_heads, int32_t q_len_max,
                                      int32_t causal, float softmax_scale, void* o, float* lse,
                                      void* workspace, int64_t workspace_bytes, int32_t dcp_world,
                                      int32_t dcp_rank, const int32_t* kv_len_global, void* stream) {
  clear_error();
  if (dcp_world < 1 || dcp_world > MLA_MAX_DCP_WORLD)
    return set_error(MLA_ERR_INVALID_ARG, "dcp_world must be in 1..64");
  if (dcp_rank < 0 || dcp_rank >= dcp_world)
    return set_error(MLA_ERR_INVALID_ARG, "dcp_rank must be in 0..dcp_world-1");
  if (!kv_len_global) return set_error(MLA_ERR_INVALID_ARG, "kv_len_global is null");
  return decode_impl(q, q_dtype, q_scale, kv_pool, kv_dtype, kv_scale, num_slots, qo_indptr,
                     kv_indptr, kv_indices, plan_host, plan_dev, rows, num_heads, q_len_max, causal,
                     softmax_scale, o, lse, workspace, workspace_bytes, stream, dcp_world, dcp_rank,
                     kv_len_global);
}

extern "C" int32_t mla_merge_shards(const void* o_parts, const float* lse_parts, int32_t world,
                                    int32_t tokens, int32_t num_heads, void* o, float* lse,
                                    void* stream) {
  clear_error();
  if (world < 1 || world > MLA_MAX_DCP_WORLD) return set_error(MLA_ERR_INVALID_ARG, "world must be in 1..64");
  if (tokens < 0 || num_heads < 1 || num_heads > MLA_MAX_HEADS)
    return set_error(MLA_ERR_INVALID_ARG, "tokens must be >= 0 and num_heads in 1..128");
  if (tokens == 0) return MLA_OK;
  if (!o_parts || !lse_parts || !o || !lse) return set_error(MLA_ERR_INVALID_ARG, "a required pointer is null");
  if (!aligned16(o_parts) || !aligned16(o)) return set_error(MLA_ERR_INVALID_ARG, "o_parts and o must be 16-byte aligned");
  ShardMergeArgs m;
  m.o_parts = (const uint16_t*)o_parts;
  m.lse_parts = lse_parts;
  m.world = world;
  m.rows = tokens * num_heads;
  m.o = (uint16_t*)o;
  m.lse = lse;
  hipError_t e = launch_shard_merge(m, (hipStream_t)stream);
  if (e != hipSuccess) return set_error(MLA_ERR_HIP, std::string("shard merge launch: ") + hipGetErrorString(e));
  return MLA_OK;
}

extern "C" int32_t mla_debug_gather(const void* kv_pool, mla_dtype kv_dtype, int64_t num_slots,
                                    const int32_t* kv_indptr, const int32_t* kv_indices,
                                    const int32_t* plan_host, const int32_t* plan_dev,
                                    int32_t rows, void* dense_out, void* stream) {
  clear_error();
  if (!kv_pool || !kv_indptr || !kv_indices || !plan_host || !dense_out)
    return set_error(MLA_ERR_INVALID_ARG, "a required pointer is null");
  if (!valid_dtype(kv_dtype)) return set_error(MLA_ERR_INVALID_ARG, "unknown kv_dtype");
  if (!aligned16(kv_pool) || !aligned16(dense_out))
    return set_error(MLA_ERR_INVALID_ARG, "kv_pool and dense_out must be 16-byte aligned");
  if (num_slots < 1 || num_slots > ((int64_t)1 << 31))
    return set_error(MLA_ERR_INVALID_ARG, "num_slots must be in 1..2^31");
  if (!plan_dev) return set_error(MLA_ERR_INVALID_ARG, "plan_dev is null");
  PlanView v;
  int32_t st = view_plan(plan_host, &v);
  if (st != MLA_OK) return st;
  if (v.rows != rows) return set_error(MLA_ERR_PLAN_MISMATCH, "plan was built for a different row count");
  if (v.kv_dtype != kv_dtype) return set_error(MLA_ERR_PLAN_MISMATCH, "plan was built for a different KV dtype");
  GatherArgs g;
  g.kv = kv_pool;
  g.kv_indptr = kv_indptr;
  g.kv_indices = kv_indices;
  g.max_slot = (uint32_t)(num_slots - 1);
  g.plan = plan_dev;
  g.off_split_row = (int32_t)v.off_split_row;
  g.off_split_begin = (int32_t)v.off_split_begin;
  g.off_split_end = (int32_t)v.off_split_end;
  g.off_split_indptr = (int32_t)v.off_split_indptr;
  g.uniform_ranges = v.mode == MLA_PLAN_UNIFORM;
  g.dense = (uint16_t*)dense_out;
  hipError_t e = launch_gather(g, kv_dtype == MLA_FP8_E4M3, v.S, (hipStream_t)stream);
  if (e != hipSuccess) return set_error(MLA_ERR_HIP, std::string("gather launch: ") + hipGetErrorString(e));
  return MLA_OK;
}

extern "C" int32_t mla_cache_write(const void* kv_c, mla_src_dtype kv_c_dtype, int64_t kv_c_stride,
                                   const void* k_pe, mla_src_dtype k_pe_dtype, int64_t k_pe_stride,
                                   const int64_t* slot_mapping, int32_t tokens, void* kv_pool,
                                   mla_dtype kv_dtype, const float* kv_scale, int64_t num_slots,
                                   void* stream) {
  clear_error();
  if (tokens < 0) return set_error(MLA_ERR_INVALID_ARG, "tokens must be >= 0");
  if (!valid_dtype(kv_dtype)) return set_error(MLA_ERR_INVALID_ARG, "unknown kv_dtype");
  auto src_size = [](int d) { return d == MLA_SRC_BF16 || d == MLA_SRC_FP16 ? 2 : d == MLA_SRC_FP32 ? 4 : 0; };
  if (!src_size(kv_c_dtype) || !src_size(k_pe_dtype))
    return set_error(MLA_ERR_INVALID_ARG, "unknown source dtype (expected MLA_SRC_BF16, MLA_SRC_FP16 or MLA_SRC_FP32)");
  if (num_slots < 1) return set_error(MLA_ERR_INVALID_ARG, "num_slots must be >= 1");
  if (kv_c_stride < 512 || k_pe_stride < 64)
    return set_error(MLA_ERR_INVALID_ARG, "kv_c_stride must be >= 512 and k_pe_stride >= 64");
  if (tokens == 0) return MLA_OK;
  if (!kv_c || !k_pe || !slot_mapping || !kv_pool)
    return set_error(MLA_ERR_INVALID_ARG, "a required pointer is null");
  if ((uintptr_t)kv_c % src_size(kv_c_dtype) || (uintptr_t)k_pe % src_size(k_pe_dtype) ||
      (uintptr_t)slot_mapping % 8 || (uintptr_t)kv_pool % 2)
    return set_error(MLA_ERR_INVALID_ARG, "a pointer is not aligned to its element size");
  CacheWriteArgs a;
  a.kv_c = kv_c;
  a.k_pe = k_pe;
  a.kv_c_dtype = kv_c_dtype;
  a.k_pe_dtype = k_pe_dtype;
  a.kv_c_stride = kv_c_stride;
  a.k_pe_stride = k_pe_stride;
  a.slots = slot_mapping;
  a.tokens = tokens;
  a.kv_fp8 = kv_dtype == MLA_FP8_E4M3;
  a.pool = kv_pool;
  a.kv_scale = kv_scale;
  a.num_slots = num_slots;
  // 8-element chunks need every row start and the pool 16-byte aligned.
  const bool vec = aligned16(kv_c) && aligned16(k_pe) && aligned16(kv_pool) &&
                   (kv_c_stride * src_size(kv_c_dtype)) % 16 == 0 &&
                   (k_pe_stride * src_size(k_pe_dtype)) % 16 == 0;
  hipError_t e = launch_cache_write(a, vec, (hipStream_t)stream);
  if (e != hipSuccess) return set_error(MLA_ERR_HIP, std::string("cache write launch: ") + hipGetErrorString(e));
  return MLA_OK;
}

extern "C" int32_t mla_decode_workspace_init(const int32_t* plan_host, void* workspace,
                                             int64_t workspace_bytes_, void* stream) {
  clear_error();
  PlanView v;
  int32_t st = view_plan(plan_host, &v);
  if (st != MLA_OK) return st;
  const int64_t need = mla::workspace_bytes(v);
  if (need == 0 || !v.merge_in_kernel) return MLA_OK;   // no counters to zero
  if (!workspace) return set_error(MLA_ERR_WORKSPACE, "this plan needs a workspace");
  if (workspace_bytes_ < need)
    return set_error(MLA_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  if (!aligned16(workspace)) return set_error(MLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  hipError_t e = launch_zero((uint32_t*)workspace, kWsCounters, (hipStream_t)stream);
  if (e != hipSuccess) return set_error(MLA_ERR_HIP, std::string("workspace init launch: ") + hipGetErrorString(e));
  return MLA_OK;
}
