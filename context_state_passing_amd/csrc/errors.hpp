// Thread-local last-error message shared by the library's entry points.
#pragma once
#include <stdarg.h>
#include <stdio.h>

#include "cpla.h"

namespace cpla {

const char* last_error_buf();
void set_error_v(const char* fmt, va_list ap);
void clear_error();

inline cpla_status fail(cpla_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  set_error_v(fmt, ap);
  va_end(ap);
  return st;
}

}  // namespace cpla
