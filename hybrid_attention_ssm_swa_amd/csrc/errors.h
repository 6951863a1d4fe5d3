// Thread-local error text shared by every entry point of the library (read
// back through hymba_last_error).
#pragma once

#include <stdint.h>

namespace hymba {

// Stores the formatted message and returns `code`.
int32_t set_error(int32_t code, const char* fmt, ...);

}  // namespace hymba
