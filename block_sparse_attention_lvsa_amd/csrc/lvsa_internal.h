// Internal helpers shared by the library's translation units (not part of the ABI).
#pragma once

#include <cstdarg>
#include <cstdint>

#include "lvsa.h"

namespace lvsa {

// Records a printf-style message as this thread's last error and returns code.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears this thread's last error; returns LVSA_OK.
int ok();

}  // namespace lvsa
