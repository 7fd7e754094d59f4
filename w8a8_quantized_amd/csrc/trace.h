// Launch trace (host side).  With SQ_TRACE set to anything other than "" or "0"
// in the environment, every kernel launch of the library writes one line to
// stderr: the kernel, its compile-time configuration (tile, waves, stages,
// rows per workgroup), the problem slice it covers and its grid.  The variable
// is read at every launch, so a process can switch the trace on and off.
#pragma once
#include <cstdio>
#include <cstdlib>

namespace sq {
inline bool trace_on() {
  const char* e = std::getenv("SQ_TRACE");
  return e && e[0] && !(e[0] == '0' && e[1] == '\0');
}
}  // namespace sq

#define SQ_TRACE(...)                                   \
  do {                                                  \
    if (::sq::trace_on()) {                             \
      std::fprintf(stderr, "sq: " __VA_ARGS__);         \
      std::fputc('\n', stderr);                         \
    }                                                   \
  } while (0)
