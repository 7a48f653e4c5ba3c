// Host-side helpers shared by the library's C ABI translation units.
#pragma once

#include "../../include/pagedkv.h"

namespace pkv {

// Record the text of a failure for pkv_last_error() on this thread and
// return st; ok() clears it and returns PKV_OK.
pkv_status fail(pkv_status st, const char* fmt, ...);
pkv_status ok();

}  // namespace pkv
