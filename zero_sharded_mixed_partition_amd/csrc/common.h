// Internal helpers shared by the host and device translation units of the
// library (not part of the public ABI).
#pragma once
#include <cstdarg>
#include <cstdint>

namespace zero_shard {

// Records a printf-style detail for zero_last_error() and returns `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

}  // namespace zero_shard
