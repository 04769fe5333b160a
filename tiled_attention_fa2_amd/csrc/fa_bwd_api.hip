// C ABI of libfa.so, backward part: argument validation and launch on the
// caller's stream. The declarations and the contract of every entry point are
// in include/fa.h.
#include <climits>
#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_api_common.hpp"
#include "fa_api_device.hpp"
#include "fa_bwd_kernel.hpp"

using fa_api::aligned16;
using fa_api::aligned4;
using fa_api::ceil_div;

namespace {

// Bytes of the (L, D) pairs, rounded up so that the dQ partials after them
// start 256-byte aligned.
size_t ld_bytes(long long BH, long long N) { return ((size_t)8 * (size_t)BH * (size_t)N + 255) & ~(size_t)255; }

// Key chunks of the dQ pass on the current device (1: no split).
int dq_splits(long long BH, long long N) {
  const int cus = fa_api::device_cus();
  return fa_api::bwd_dq_splits(BH * ceil_div(N, fa::bwd::kRows), N, cus);
}

}  // namespace

extern "C" size_t fa_bwd_workspace_bytes(int B, int H, int N) {
  if (B < 0 || H < 0 || N < 0) return 0;
  const long long BH = (long long)B * H;
  const int S = dq_splits(BH, N);
  if (S <= 1) return (size_t)8 * (size_t)BH * (size_t)N;
  // the dQ partials, sized for head dim 128
  return ld_bytes(BH, N) + (size_t)S * (size_t)BH * (size_t)N * 128 * 4;
}

// 32-key blocks per wave of the dK/dV kernel (each wave reads its Q / dO
// operands once for all of them): two at both head dims; at 128 the second
// block's K/V operands are staged in LDS (its accumulators fill the registers)
#ifndef FA_DKDV_KB
#define FA_DKDV_KB 2
#endif
constexpr int kDkdvKB = FA_DKDV_KB;

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                      int d, int causal, float scale, int dtype, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || Hq < 0 || N < 0) return FA_ERR_SHAPE;
  if (Hq > 0 && (Hkv < 1 || Hq % Hkv != 0)) return FA_ERR_SHAPE;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  const long long BH = (long long)B * Hq;
  if (BH == 0 || N == 0) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_ALIGN;
  if (!workspace || !aligned16(workspace) || workspace_bytes < fa_bwd_workspace_bytes(B, Hq, N))
    return FA_ERR_WORKSPACE;
  const long long n_tiles = ceil_div(N, fa::bwd::kRows);
  if (BH > INT_MAX || BH * n_tiles > INT_MAX) return FA_ERR_SHAPE;
  if (((long long)N + 128) * d * 2 > INT_MAX) return FA_ERR_SHAPE;
  const long long pre_blocks = ceil_div(BH * N, 256 / (d / 8));
  if (pre_blocks > INT_MAX) return FA_ERR_SHAPE;

  fa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.ld = static_cast<float2*>(workspace);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.BH = (int)BH;
  a.N = N;
  a.group = Hq / Hkv;
  a.n_tiles = (int)n_tiles;
  // one key block per wave when two would leave compute units idle: twice the
  // workgroups, each reading its Q / dO operands for one block (measured:
  // 8 heads x 4096 tokens, 128 workgroups of two blocks against 256 of one)
  const int cus = fa_api::device_cus();
  const bool one_block = kDkdvKB == 2 && cus > 0 && (BH / a.group) * ceil_div(N, fa::bwd::kRows * 2) < cus;
  a.n_ktiles = (int)ceil_div(N, fa::bwd::kRows * (one_block ? 1 : kDkdvKB));
  a.causal_order = fa_api::causal_order(BH, a.group, N, d, 2);
  // a dK/dV item (one key/value head) streams the Q and dO rows of its
  // `group` query heads: the same rule with group * d bytes per row
  a.causal_order_kv = fa_api::causal_order(BH / a.group, 1, N, (long long)d * a.group, 2);
  a.scale = scale;
  // dQ key split on grids that leave the SIMDs with fewer than two waves
  const int S = dq_splits(BH, N);
  a.dq_splits = S;
  a.dq_chunk_tiles = (int)ceil_div(ceil_div(N, 32), S);
  a.dq_part = S > 1 ? reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + ld_bytes(BH, N)) : nullptr;
  if (BH * n_tiles * S > INT_MAX) return FA_ERR_SHAPE;
  const long long merge_blocks = ceil_div(BH * N, 256 / (d / 8));
  const dim3 blk(256), g_pre((unsigned)pre_blocks), g_dq((unsigned)(BH * n_tiles * S)),
      g_dkdv((unsigned)(BH / a.group * a.n_ktiles)), g_merge((unsigned)merge_blocks);
  const bool c = causal != 0;
  const bool split = S > 1;
  if (d == 128) {
    hipLaunchKernelGGL(fa::fa_bwd_pre_kernel<128>, g_pre, blk, 0, stream, a);
    if (c) {
      if (one_block)
        hipLaunchKernelGGL((fa::fa_bwd_dkdv_kernel<128, true, 1, 1>), g_dkdv, blk, 0, stream, a);
      else
        hipLaunchKernelGGL((fa::fa_bwd_dkdv_kernel<128, true, kDkdvKB, 1>), g_dkdv, blk, 0, stream, a);
      if (split) {
        hipLaunchKernelGGL((fa::fa_bwd_dq_kernel<128, true, true>), g_dq, blk, 0, stream, a);
        hipLaunchKernelGGL(fa::fa_bwd_dq_merge_kernel<128>, g_merge, blk, 0, stream, a);
      } else {
        hipLaunchKernelGGL((fa::fa_bwd_dq_kernel<128, true>), g_dq, blk, 0, stream, a);
      }
    } else {
      if (one_block)
        hipLaunchKernelGGL((fa::fa_bwd_dkdv_kernel<128, false, 1, 1>), g_dkdv, blk, 0, stream, a);
      else
        hipLaunchKernelGGL((fa::fa_bwd_dkdv_kernel<128, false, kDkdvKB, 1>), g_dkdv, blk, 0, stream, a);
      if (split) {
        hipLaunchKernelGGL((fa::fa_bwd_dq_kernel<128, false, true>), g_dq, blk, 0, stream, a);
        hipLaunchKernelGGL(fa::fa_bwd_dq_merge_kernel<128>, g_merge, blk, 0, stream, a);
      } else {
        hipLaunchKernelGGL((fa::fa_bwd_dq_kernel<128, false>), g_dq, blk, 0, stream, a);
      }
    }
  } else {
    hipLaunchKernelGGL(fa::fa_bwd_pre_kernel<64>, g_pre, blk, 0, stream, a);
    if (c) {
      if (one_block)
        hipLaunchKernelGGL((fa::fa_bwd_dkdv_kernel<64, true, 1, 1>), g_dkdv, blk, 0, stream, a);
      else
        hipLaunchKernelGGL((fa::fa_bwd_dkdv_kernel<64, true, kDkdvKB, kDkdvKB>), g_dkdv, blk, 0, stream, a);
      if (split) {
        hipLaunchKernelGGL((fa::fa_bwd_dq_kernel<64, true, true>), g_dq, blk, 0, stream, a);
        hipLaunchKernelGGL(fa::fa_bwd_dq_merge_kernel<64>, g_merge, blk, 0, stream, a);
      } else {
        hipLaunchKernelGGL((fa::fa_bwd_dq_kernel<64, true>), g_dq, blk, 0, stream, a);
      }
    } else {
      if (one_block)
        hipLaunchKernelGGL((fa::fa_bwd_dkdv_kernel<64, false, 1, 1>), g_dkdv, blk, 0, stream, a);
      else
        hipLaunchKernelGGL((fa::fa_bwd_dkdv_kernel<64, false, kDkdvKB, kDkdvKB>), g_dkdv, blk, 0, stream, a);
      if (split) {
        hipLaunchKernelGGL((fa::fa_bwd_dq_kernel<64, false, true>), g_dq, blk, 0, stream, a);
        hipLaunchKernelGGL(fa::fa_bwd_dq_merge_kernel<64>, g_merge, blk, 0, stream, a);
      } else {
        hipLaunchKernelGGL((fa::fa_bwd_dq_kernel<64, false>), g_dq, blk, 0, stream, a);
      }
    }
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
