// internal.h -- shared helpers of libsnack_coo (not part of the public ABI).
#pragma once

#include <cstdarg>
#include <cstdint>

namespace snack {

// Records a printf-style message for snack_last_error() and returns `status`.
int fail(int status, const char *fmt, ...);
// Clears the calling thread's message and returns SNACK_OK.
int ok();

// Process-wide kernel-selection override set by snack_coo_set_option (SNACK_OPT_*); -1 means
// the library's own choice.
int64_t option(int which);

}  // namespace snack
