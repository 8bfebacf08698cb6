// Thread-local error state of the C ABI.
#pragma once

#include "../../include/bac.h"

namespace bac {

void clear_error();
// printf-style message; returns `code` so callers can `return fail(...)`.
bac_status fail(bac_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace bac
