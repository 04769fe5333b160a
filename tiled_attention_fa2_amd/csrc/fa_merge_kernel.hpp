// Merge of split-KV partial results for gfx950.
//
// "Kernels and Memory in LLM Inference", section "Flash-Decoding: one token,
// whole chip": every key chunk's attention is formed on its own, with its own
// max and sum, and a second small kernel merges the partials by rescaling each
// to the overall max. A partial here is the chunk's output already divided by
// its own sum, O_s, with its natural-log logsumexp L_s; rescaling chunk s to a
// common max M weighs it by exp(L_s - M), so per query row
//     M = max_s L_s,  w_s = exp(L_s - M),  O = sum_s w_s O_s / sum_s w_s,
//     L = M + log sum_s w_s,
// and chunks with L_s = -inf (no valid key) weigh nothing.
//
// The work is HBM-bound (read S rows of fp32 partials, write one output row):
// d/4 lanes per row, one float4 of every partial per lane, coalesced.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// two floats -> one dword of two bf16 (round to nearest even), low half first
__device__ __forceinline__ uint32_t merge_pack_bf16(float lo, float hi) {
  typedef float m_f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 m_bf16x2 __attribute__((ext_vector_type(2)));
  const m_f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, m_bf16x2));
}

// One row of the merge: lane c4 (of D/4) of row `row` (of `rows`).
template <int D, bool OUT_F32>
__device__ __forceinline__ void merge_row(const float* __restrict__ o_part, const float* __restrict__ lse_part,
                                          int S, long long rows, long long row, int c4, void* __restrict__ o,
                                          float* __restrict__ lse) {
  float M = -__builtin_inff();
  for (int s = 0; s < S; ++s) M = fmaxf(M, lse_part[(size_t)s * rows + row]);
  float z = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (M > -__builtin_inff()) {
    for (int s = 0; s < S; ++s) {
      const float Ls = lse_part[(size_t)s * rows + row];
      if (Ls == -__builtin_inff()) continue;
      const float w = expf(Ls - M);
      const float4 x = ((const float4*)(o_part + ((size_t)s * rows + row) * D))[c4];
      z += w;
      acc.x += w * x.x;
      acc.y += w * x.y;
      acc.z += w * x.z;
      acc.w += w * x.w;
    }
  }
  const float inv = z > 0.0f ? 1.0f / z : 0.0f;
  if constexpr (OUT_F32) {
    ((float4*)((float*)o + (size_t)row * D))[c4] =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  } else {
    uint2 pk;
    pk.x = merge_pack_bf16(acc.x * inv, acc.y * inv);
    pk.y = merge_pack_bf16(acc.z * inv, acc.w * inv);
    ((uint2*)((unsigned short*)o + (size_t)row * D))[c4] = pk;
  }
  if (c4 == 0) lse[row] = z > 0.0f ? M + logf(z) : -__builtin_inff();
}

// o_part [S][rows][D], lse_part [S][rows] -> o [rows][D] (fp32 or bf16), lse [rows]
template <int D, bool OUT_F32>
__global__ void __launch_bounds__(256) fa_merge_kernel(const float* __restrict__ o_part,
                                                       const float* __restrict__ lse_part, int S,
                                                       long long rows, void* __restrict__ o,
                                                       float* __restrict__ lse) {
  constexpr int TPR = D / 4;          // lanes per row
  constexpr int RPB = 256 / TPR;      // rows per workgroup
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= rows) return;
  merge_row<D, OUT_F32>(o_part, lse_part, S, rows, row, threadIdx.x % TPR, o, lse);
}

}  // namespace fa
