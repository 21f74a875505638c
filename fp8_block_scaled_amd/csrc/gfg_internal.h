// Internal declarations shared by the host and device halves of libgfg.
#pragma once
#include <cstdint>

namespace gfg {
// Record a formatted message as the calling thread's last error; returns code.
int fail(int code, const char* fmt, ...);
void clear_error();
}  // namespace gfg
