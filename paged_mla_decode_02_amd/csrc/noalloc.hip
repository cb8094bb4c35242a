// mla_decode_fwd_noalloc: the decode with the split partials (and, for an
// in-kernel-merge plan, the split-arrival counters) in a library-owned static
// device array instead of a caller workspace, for callers that cannot
// allocate device memory (code under graph capture, serving loops that may
// not call the allocator, harnesses that forbid it).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends. In host code the
// array's name is only a host-side stand-in, so its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and only
// that address is ever passed to a kernel. Every call on one GPU shares that
// GPU's array and leaves the last call's partials in it, so calls that
// overlap on one GPU (concurrent streams, threads) race.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <mutex>
#include <string>

#include "kernel_args.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int64_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];   // device address of `scratch` per device, once looked up

// Device address of the current device's copy of `scratch` (looked up on the
// first call made with that device current).
int32_t current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(MLA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_error(MLA_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(MLA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MLA_OK;
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" int32_t mla_decode_fwd_noalloc(const void* q, mla_dtype q_dtype, const float* q_scale,
                                          const void* kv_pool, mla_dtype kv_dtype,
                                          const float* kv_scale, int64_t num_slots,
                                          const int32_t* qo_indptr, const int32_t* kv_indptr,
                                          const int32_t* kv_indices, const int32_t* plan_host,
                                          const int32_t* plan_dev, int32_t rows, int32_t num_heads,
                                          int32_t q_len_max, int32_t causal, float softmax_scale,
                                          void* o, float* lse, void* stream) {
  clear_error();
  PlanView v;
  int32_t st = view_plan(plan_host, &v);
  if (st != MLA_OK) return st;
  const int64_t need = workspace_bytes(v);
  if (need > kScratchBytes)
    return set_error(MLA_ERR_WORKSPACE, "this plan needs " + std::to_string(need) +
                                            " bytes of scratch; the static scratch holds " +
                                            std::to_string(kScratchBytes) +
                                            " (use mla_decode_fwd with a caller workspace)");
  void* ws = nullptr;
  if (need > 0) {
    st = current_scratch(&ws);
    if (st != MLA_OK) return st;
  }
  // The split-arrival counters of an in-kernel-merge plan must start at zero:
  // decode_impl clears the ones this call can touch with a fill kernel (not
  // a memset, so the call may be captured in a graph).
  return decode_impl(q, q_dtype, q_scale, kv_pool, kv_dtype, kv_scale, num_slots, qo_indptr,
                     kv_indptr, kv_indices, plan_host, plan_dev, rows, num_heads, q_len_max, causal,
                     softmax_scale, o, lse, ws, need > 0 ? kScratchBytes : 0, stream, 1, 0, nullptr,
                     /*clear_counters=*/true);
}
