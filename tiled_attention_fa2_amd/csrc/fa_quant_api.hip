// C ABI of libfa.so, FP8 quantiser part: argument validation and launch on the
// caller's stream. The declarations and the contract of every entry point are
// in include/fa.h.
#include <climits>
#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_api_common.hpp"
#include "fa_quant_kernel.hpp"

using fa_api::aligned16;
using fa_api::aligned4;
using fa_api::ceil_div;

extern "C" int fa_quantize_fp8(const void* x, int in_dtype, void* x_fp8, float* descale,
                               int B, int H, int N, int d, hipStream_t stream) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (in_dtype != FA_DTYPE_F32 && in_dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  const long long BH = (long long)B * H;
  if (BH == 0) return FA_OK;
  if (!descale) return FA_ERR_NULL;
  if (BH > 65535) return FA_ERR_SHAPE;  // grid.y limit of the per-head kernels
  if (N > 0 && (!x || !x_fp8)) return FA_ERR_NULL;
  if (N > 0 && (!aligned16(x) || !aligned16(x_fp8))) return FA_ERR_ALIGN;
  uint32_t* amax = reinterpret_cast<uint32_t*>(descale);
  const int nbh = (int)BH;
  const long long per_head = (long long)N * d;

  hipLaunchKernelGGL(fa::fa_amax_clear, dim3((nbh + 255) / 256), dim3(256), 0, stream, amax, nbh);
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  if (N > 0) {
    // about 64 elements per thread per workgroup pass, at most 256 workgroups per head
    long long bph = (per_head / 16 + 256 * 4 - 1) / (256 * 4);
    if (bph < 1) bph = 1;
    if (bph > 256) bph = 256;
    const dim3 grid((unsigned)bph, (unsigned)nbh);
    // the amax pass reads only: a quarter of the workgroups, each streaming
    // four times as much (measured 131 -> 100 us on a 56 x 30272 x 128 tensor)
    const dim3 grid_a((unsigned)((bph + 3) / 4), (unsigned)nbh);
    if (in_dtype == FA_DTYPE_BF16) {
      hipLaunchKernelGGL(fa::fa_amax_kernel<true>, grid_a, dim3(256), 0, stream, x, amax, per_head);
      hipLaunchKernelGGL(fa::fa_quant_kernel<true>, grid, dim3(256), 0, stream, x,
                         (uint8_t*)x_fp8, (const uint32_t*)amax, per_head);
    } else {
      hipLaunchKernelGGL(fa::fa_amax_kernel<false>, grid_a, dim3(256), 0, stream, x, amax, per_head);
      hipLaunchKernelGGL(fa::fa_quant_kernel<false>, grid, dim3(256), 0, stream, x,
                         (uint8_t*)x_fp8, (const uint32_t*)amax, per_head);
    }
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  }
  hipLaunchKernelGGL(fa::fa_descale_finalize, dim3((nbh + 255) / 256), dim3(256), 0, stream, amax,
                     nbh);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_quantize_fp8_rotated(const void* x, int in_dtype, const signed char* signs,
                                       void* x_fp8, float* descale, int B, int H, int N, int d,
                                       int fold_inverse_d, hipStream_t stream) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (in_dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  const long long BH = (long long)B * H;
  if (BH == 0) return FA_OK;
  if (!descale || !signs) return FA_ERR_NULL;
  if (BH > 65535) return FA_ERR_SHAPE;  // grid.y limit of the per-head kernels
  if (N > 0 && (!x || !x_fp8)) return FA_ERR_NULL;
  if (N > 0 && (!aligned16(x) || !aligned16(x_fp8))) return FA_ERR_ALIGN;
  uint32_t* amax = reinterpret_cast<uint32_t*>(descale);
  const int nbh = (int)BH;

  hipLaunchKernelGGL(fa::fa_amax_clear, dim3((nbh + 255) / 256), dim3(256), 0, stream, amax, nbh);
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  if (N > 0) {
    // d/32 lanes per row; about 2 rows per lane, at most 256 workgroups per head
    const int rows_per_block = 256 / (d / 32);
    long long bph = ((long long)N + rows_per_block * 2 - 1) / (rows_per_block * 2);
    if (bph > 256) bph = 256;
    const dim3 grid((unsigned)bph, (unsigned)nbh);
    if (d == 128) {
      hipLaunchKernelGGL(fa::fa_rot_amax_kernel<128>, grid, dim3(256), 0, stream, x, signs, amax, N);
      hipLaunchKernelGGL(fa::fa_rot_quant_kernel<128>, grid, dim3(256), 0, stream, x, signs,
                         (uint8_t*)x_fp8, (const uint32_t*)amax, N);
    } else {
      hipLaunchKernelGGL(fa::fa_rot_amax_kernel<64>, grid, dim3(256), 0, stream, x, signs, amax, N);
      hipLaunchKernelGGL(fa::fa_rot_quant_kernel<64>, grid, dim3(256), 0, stream, x, signs,
                         (uint8_t*)x_fp8, (const uint32_t*)amax, N);
    }
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  }
  const float post = fold_inverse_d ? 1.0f / (float)d : 1.0f;
  hipLaunchKernelGGL(fa::fa_descale_finalize_scaled, dim3((nbh + 255) / 256), dim3(256), 0, stream,
                     amax, nbh, post);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_quantize_mxfp8_rows(const void* x, int in_dtype, const signed char* signs,
                                      int fold_inverse_d, void* x_fp8, unsigned char* scales, int B,
                                      int H, int N, int d, hipStream_t stream) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (in_dtype != FA_DTYPE_F32 && in_dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (signs && in_dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  const long long BH = (long long)B * H;
  if (BH == 0 || N == 0) return FA_OK;
  if (!x || !x_fp8 || !scales) return FA_ERR_NULL;
  if (!aligned16(x) || !aligned16(x_fp8)) return FA_ERR_ALIGN;
  const float post = fold_inverse_d ? 1.0f / (float)d : 1.0f;
  if (!signs) {
    const long long nblocks = BH * N * (d / 32);
    const long long grid = ceil_div(nblocks, 256);
    if (grid > INT_MAX) return FA_ERR_SHAPE;
    if (in_dtype == FA_DTYPE_BF16)
      hipLaunchKernelGGL(fa::fa_mx_rows_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, x,
                         (uint8_t*)x_fp8, scales, nblocks, post);
    else
      hipLaunchKernelGGL(fa::fa_mx_rows_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, x,
                         (uint8_t*)x_fp8, scales, nblocks, post);
  } else {
    if (BH > 65535) return FA_ERR_SHAPE;   // grid.y limit of the per-head kernel
    // d/32 lanes per row; about 2 rows per lane, at most 256 workgroups per head
    const int rows_per_block = 256 / (d / 32);
    long long bph = ceil_div(N, rows_per_block * 2);
    if (bph > 256) bph = 256;
    const dim3 grid((unsigned)bph, (unsigned)BH);
    if (d == 128)
      hipLaunchKernelGGL(fa::fa_mx_rows_rot_kernel<128>, grid, dim3(256), 0, stream, x, signs,
                         (uint8_t*)x_fp8, scales, N, post);
    else
      hipLaunchKernelGGL(fa::fa_mx_rows_rot_kernel<64>, grid, dim3(256), 0, stream, x, signs,
                         (uint8_t*)x_fp8, scales, N, post);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_quantize_mxfp8_keys(const void* x, int in_dtype, void* x_fp8, unsigned char* scales,
                                      int B, int H, int N, int d, hipStream_t stream) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (in_dtype != FA_DTYPE_F32 && in_dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  const long long BH = (long long)B * H;
  if (BH == 0 || N == 0) return FA_OK;
  if (!x || !x_fp8 || !scales) return FA_ERR_NULL;
  if (!aligned16(x) || !aligned16(x_fp8) || !aligned4(scales)) return FA_ERR_ALIGN;
  const int nkb = (int)ceil_div(N, 32);
  const long long items = BH * nkb * (d / 4);
  const long long grid = ceil_div(items, 256);
  if (grid > INT_MAX) return FA_ERR_SHAPE;
  const dim3 g((unsigned)grid), blk(256);
  if (in_dtype == FA_DTYPE_BF16) {
    if (d == 128)
      hipLaunchKernelGGL((fa::fa_mx_keys_kernel<true, 128>), g, blk, 0, stream, x, (uint8_t*)x_fp8, scales, N,
                         nkb, items);
    else
      hipLaunchKernelGGL((fa::fa_mx_keys_kernel<true, 64>), g, blk, 0, stream, x, (uint8_t*)x_fp8, scales, N,
                         nkb, items);
  } else {
    if (d == 128)
      hipLaunchKernelGGL((fa::fa_mx_keys_kernel<false, 128>), g, blk, 0, stream, x, (uint8_t*)x_fp8, scales,
                         N, nkb, items);
    else
      hipLaunchKernelGGL((fa::fa_mx_keys_kernel<false, 64>), g, blk, 0, stream, x, (uint8_t*)x_fp8, scales,
                         N, nkb, items);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
