// Small helpers shared by the C-ABI source files of libfa.so.
#pragma once

#include <cstdint>

namespace fa_api {

inline long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace fa_api
