// status.h -- the library's error text (lca_last_error), shared by the C ABI sources.
#pragma once

namespace lca {
// records the message (printf format) for lca_last_error() and returns code
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
}  // namespace lca
