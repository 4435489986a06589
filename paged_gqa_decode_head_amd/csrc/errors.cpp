#include "errors.hpp"

#include <cstdarg>
#include <cstdio>

namespace pgqa {
namespace {
thread_local char g_err[512] = "";
}

pgqa_status fail(pgqa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = 0; }

const char* last_error() { return g_err; }

}  // namespace pgqa
