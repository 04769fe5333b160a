// Small helpers shared by the C-ABI source files of libfa.so.
#pragma once

#include <cstdint>

namespace fa_api {

inline long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Order of causal work items (the kernels' work_item): 2, longest query tiles
// first across the heads one XCD holds, when the heads split evenly over the 8
// XCDs and the distinct K/V bytes of one XCD's heads stay within 32 MiB (the
// tail of short causal problems shrinks; measured +10% at 4 x 32 x 2048 bf16);
// else 1, head by head, which keeps one head's K/V stream in the XCD's L2 on
// long sequences (interleaving 7 heads of 30272 tokens lost 4.5%).
inline int causal_order(long long BH, long long group, long long N, long long d, long long es) {
  if (BH % 8 != 0 || group < 1) return 1;
  const long long heads = BH / 8;
  const long long kv_heads = (heads + group - 1) / group + (heads % group != 0 ? 1 : 0);
  return kv_heads * 2 * N * d * es <= (32ll << 20) ? 2 : 1;
}

}  // namespace fa_api
