// Thread-local error text behind wf_last_error(). Host only.
#pragma once
#include <cstdarg>
#include <cstdint>

namespace wf {
// Records printf-style text for wf_last_error() and returns `status`.
int32_t fail(int32_t status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
}  // namespace wf
