// Status reporting shared by the C ABI's translation units: a failing check records
// its detail for pkv_last_error (per thread) and returns its pkv_status.
#pragma once

namespace pkv {

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace pkv
