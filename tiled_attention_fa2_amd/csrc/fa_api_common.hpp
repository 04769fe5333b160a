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

// Number of key chunks for the split-KV forward on a device with `cus`
// compute units, given wgs = B*H*ceil(N/128) unsplit workgroups: none once
// there are two workgroups per CU; else enough chunks for about two per CU
// (non-causal) or three (causal, whose uneven per-tile work needs more pieces
// to balance), never a chunk under 1024 keys, nor, when a non-causal grid
// already has a workgroup on every CU, under 2048 (bf16) or 4096 (FP8) keys;
// at most 16. Measured on MI355X (bf16 and FP8 at d = 128, bf16 at d = 64):
// filling every slot instead cost up to 26% (32 heads x 1024 tokens, chunks of
// 341 keys), splitting 512 workgroups cost 7-11%, 16 x 2048 lost 3.6% with
// chunks of 1024 keys, and FP8 8 x 4096 (wide tiles unsplit) 5% in 2 chunks.
inline int default_splits(long long wgs, long long N, bool causal, long long cus, bool fp8 = false) {
  if (wgs <= 0 || N <= 0 || cus <= 0 || wgs >= 2 * cus) return 1;
  long long s = ceil_div((causal ? 3 : 2) * cus, wgs);
  const long long min_keys = (!causal && wgs >= cus) ? (fp8 ? 4096 : 2048) : 1024;
  const long long by_keys = N / min_keys > 1 ? N / min_keys : 1;
  if (s > by_keys) s = by_keys;
  if (s > 16) s = 16;
  return (int)(s < 1 ? 1 : s);
}

// Key chunks of the backward's dQ pass, given its wgs = B*H*ceil(N/128)
// workgroups and the device's CUs: one when the grid already gives every CU
// two workgroups (two waves per SIMD, what the dQ kernel is built for); else
// the fewest chunks that reach two per CU, no chunk under 1024 keys, at most 8.
// The partial dQ of every chunk goes through the workspace
// (fa_bwd_workspace_bytes).
#ifndef FA_DQ_MAX_SPLITS
#define FA_DQ_MAX_SPLITS 8
#endif
inline int bwd_dq_splits(long long wgs, long long N, long long cus) {
  if (wgs <= 0 || N <= 0 || cus <= 0 || wgs >= 2 * cus) return 1;
  long long s = ceil_div(2 * cus, wgs);
  const long long by_keys = N / 1024 > 1 ? N / 1024 : 1;
  if (s > by_keys) s = by_keys;
  if (s > FA_DQ_MAX_SPLITS) s = FA_DQ_MAX_SPLITS;
  return (int)(s < 1 ? 1 : s);
}

}  // namespace fa_api
