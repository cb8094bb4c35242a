// Thread-local error message and version query.
#include <string>

#include "mla_internal.h"

namespace mla {
namespace {
thread_local std::string g_last_error;
}

int32_t set_error(int32_t status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

void clear_error() { g_last_error.clear(); }

}  // namespace mla

extern "C" const char* mla_last_error(void) { return mla::g_last_error.c_str(); }

extern "C" int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }
