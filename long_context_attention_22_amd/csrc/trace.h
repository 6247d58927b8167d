// trace.h -- call tracing.  With the environment variable LCA_TRACE set (to anything but "0"),
// every C-ABI call logs one line to stderr with its shapes, formats and first position, every
// error its code and message, and the attention, compressor and linear-map launches their kernel
// and grid.  Lines start with "[lca]"; the flag is read once per process.
#pragma once

namespace lca {
bool trace_on();
void trace(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
}  // namespace lca
