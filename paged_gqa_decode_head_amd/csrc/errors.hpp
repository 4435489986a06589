// Thread-local error message of the C ABI (pgqa_last_error).
#pragma once

#include "../../include/pgqa.h"

namespace pgqa {

// Records a printf-style message for pgqa_last_error() and returns s.
pgqa_status fail(pgqa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the message at the start of a call.
void clear_error();
const char* last_error();

}  // namespace pgqa
