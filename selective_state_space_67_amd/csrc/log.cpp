// Launch log (log.h): one flag read from the environment once per process,
// lines written to stderr with a single call each so that threads do not
// interleave inside a line.
#include "log.h"

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace ssm {

bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("SSM_LOG");
    return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
  }();
  return on;
}

void log_printf(const char* fmt, ...) {
  char line[512];
  int n = std::snprintf(line, sizeof(line), "[ssm] ");
  va_list ap;
  va_start(ap, fmt);
  const int m = std::vsnprintf(line + n, sizeof(line) - n - 1, fmt, ap);
  va_end(ap);
  n = m < 0 ? n : std::min<int>(n + m, static_cast<int>(sizeof(line)) - 2);
  line[n] = '\n';
  line[n + 1] = '\0';
  std::fputs(line, stderr);
}

}  // namespace ssm
