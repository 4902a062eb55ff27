// Per-thread error message of the C ABI (read back through pa_last_error), shared by the
// translation units that implement entry points.
#pragma once

#include "pagedattn.h"

namespace pa {

// Record a formatted message for this thread and return `st`.
pa_status fail(pa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear this thread's message and return PA_OK.
pa_status ok();
const char* last_error();

}  // namespace pa
