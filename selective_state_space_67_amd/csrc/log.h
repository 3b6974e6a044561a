// Launch log of libssmscan.so.
//
// With the environment variable SSM_LOG set to anything but "" or "0" (read
// once, on the library's first log call), every entry point prints its plan
// (sizes, pieces the sequence is split into, workspace) and every kernel
// launch prints the kernel with its tile, grid and block, one line each to
// stderr, prefixed "[ssm]". Unset, a call costs one load of a cached flag.
#pragma once

namespace ssm {

bool log_enabled();
void log_printf(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

}  // namespace ssm

#define SSM_LOG(...)                                           \
  do {                                                         \
    if (::ssm::log_enabled()) ::ssm::log_printf(__VA_ARGS__);  \
  } while (0)
