// Host-only internals shared by the library's C ABI sources.
#pragma once
#include <string>

#include "zero_shard.h"

namespace zs {

// Sets the calling thread's message for zero_last_error() and returns s.
zero_status_t set_error(zero_status_t s, const std::string& msg);

}  // namespace zs
