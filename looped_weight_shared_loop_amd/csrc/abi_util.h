// Error reporting shared by the C ABI translation units.
#pragma once
#include <cstdint>

// Records a message for loop_last_error() (thread-local) and returns `code`.
int lp_fail(int code, const char* fmt, ...);

inline bool lp_misaligned(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
