// internal.h -- shared helpers of libsnack_coo (not part of the public ABI).
#pragma once

#include <cstdarg>
#include <cstdint>

namespace snack {

// Records a printf-style message for snack_last_error() and returns `status`.
int fail(int status, const char *fmt, ...);
// Clears the calling thread's message and returns SNACK_OK.
int ok();

}  // namespace snack
