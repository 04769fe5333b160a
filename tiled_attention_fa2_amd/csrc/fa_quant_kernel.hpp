// Per-head FP8-e4m3 quantisation for gfx950.
//
// "1.8x Faster Attention on an RTX 5080" (section "Who am I, what's mine?")
// feeds its kernel FP8 Q, K and V with one fp32 descale per head. Per
// (batch, head): amax = max |x|; descale = amax / 448; code =
// e4m3(clamp(x * 448 / amax, -448, 448)), rounded to nearest even. An all-zero
// head gets descale 1.
//
// The work is HBM-bound (read 2 or 4 bytes, write 1 byte per element), so the
// kernels are plain streaming loops: 16 elements per thread per step with
// 16-byte vector loads and stores, many workgroups per head, and the per-head
// amax combined with one atomic max per workgroup on the float's bit pattern
// (non-negative floats order like their unsigned bit patterns).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef unsigned int qu32x4 __attribute__((ext_vector_type(4)));

// 32-bit reinterpretations taking their argument by value (see f2u / u2f in
// the forward kernel: bit-casting an ext_vector element in place is unsafe).
__device__ __forceinline__ float q_u2f(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t q_f2u(float x) { return __builtin_bit_cast(uint32_t, x); }

__global__ void fa_amax_clear(uint32_t* amax_bits, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) amax_bits[i] = 0u;
}

// Load 16 consecutive elements starting at element `e` as floats.
template <bool BF16>
__device__ __forceinline__ void load16(const void* base, size_t e, float* out) {
  if constexpr (BF16) {
    const qu32x4* src = (const qu32x4*)((const unsigned short*)base + e);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const qu32x4 w = src[h];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        out[8 * h + 2 * k] = q_u2f(w[k] << 16);
        out[8 * h + 2 * k + 1] = q_u2f(w[k] & 0xffff0000u);
      }
    }
  } else {
    const qu32x4* src = (const qu32x4*)((const float*)base + e);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const qu32x4 w = src[h];
#pragma unroll
      for (int k = 0; k < 4; ++k) out[4 * h + k] = q_u2f(w[k]);
    }
  }
}

// grid = (blocks per head, B*H); per_head = N*d elements, a multiple of 16.
template <bool BF16>
__global__ void __launch_bounds__(256) fa_amax_kernel(const void* x, uint32_t* amax_bits,
                                                      long long per_head) {
  const int bh = blockIdx.y;
  const size_t head0 = (size_t)bh * (size_t)per_head;
  const long long n16 = per_head / 16;
  float m = 0.0f;
  for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < n16;
       t += (long long)gridDim.x * blockDim.x) {
    float v[16];
    load16<BF16>(x, head0 + (size_t)t * 16, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  // wave reduction, then one value per wave through LDS
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float b = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    atomicMax(amax_bits + bh, q_f2u(b));
  }
}

template <bool BF16>
__global__ void __launch_bounds__(256) fa_quant_kernel(const void* x, uint8_t* out,
                                                       const uint32_t* amax_bits,
                                                       long long per_head) {
  const int bh = blockIdx.y;
  const float amax = q_u2f(amax_bits[bh]);
  // correctly rounded fp32 division (no fast-math anywhere in this library)
  const float mult = amax == 0.0f ? 1.0f : 448.0f / amax;
  const size_t head0 = (size_t)bh * (size_t)per_head;
  const long long n16 = per_head / 16;
  for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < n16;
       t += (long long)gridDim.x * blockDim.x) {
    float v[16];
    load16<BF16>(x, head0 + (size_t)t * 16, v);
    qu32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float y[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) y[k] = fminf(fmaxf(v[4 * w + k] * mult, -448.0f), 448.0f);
      int pk = 0;
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], pk, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], pk, true);
      o[w] = (uint32_t)pk;
    }
    *(qu32x4*)(out + head0 + (size_t)t * 16) = o;
  }
}

// ---------------------------------------------------------------------------
// Rotation before quantisation ("Kernels and Memory in LLM Inference", section
// "Precision: FP8 with a real failure mode": Q and K are multiplied by a fixed
// random rotation before FP8 quantisation, which spreads outlier coordinates;
// the rotations cancel in Q K^T). Here the rotation is the randomised Hadamard
// transform y = (x * s) H (s: d signs, H: the unnormalised Sylvester matrix,
// H H^T = d I), computed as a fast Walsh-Hadamard transform in float64: every
// partial sum of at most d signed bf16 values is exact there (unless a row
// spans more than 38 binary orders of magnitude), so y is the exact sum
// rounded once to fp32 whatever the order. Each row of D bf16 is handled by
// D/8 consecutive lanes holding 8 consecutive elements each: butterflies of
// stride 1, 2, 4 inside a lane, 8..D/2 across lanes.
template <int D>
__device__ __forceinline__ void rotate_row8(const void* x, size_t e0, const signed char* signs, int c,
                                            float* y) {
  const qu32x4 w = *(const qu32x4*)((const unsigned short*)x + e0);
  double v[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = (double)q_u2f(w[k] << 16);
    v[2 * k + 1] = (double)q_u2f(w[k] & 0xffff0000u);
  }
#pragma unroll
  for (int t = 0; t < 8; ++t)
    if (signs[8 * c + t] < 0) v[t] = -v[t];
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if ((t & h) == 0) {
        const double a = v[t], b = v[t + h];
        v[t] = a + b;
        v[t + h] = a - b;
      }
#pragma unroll
  for (int m = 1; m < D / 8; m <<= 1) {
    const bool upper = (c & m) != 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const double other = __shfl_xor(v[t], m);
      v[t] = upper ? other - v[t] : v[t] + other;
    }
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) y[t] = (float)v[t];
}

// grid = (blocks per head, B*H); rows of D bf16, D/8 lanes per row
template <int D>
__global__ void __launch_bounds__(256) fa_rot_amax_kernel(const void* x, const signed char* signs,
                                                          uint32_t* amax_bits, int N) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;
  const int bh = blockIdx.y;
  const int c = threadIdx.x % TPR;
  float m = 0.0f;
  // every lane runs the same trip count so that the row's shuffles stay whole
  for (int r0 = blockIdx.x * RPB; r0 < N; r0 += gridDim.x * RPB) {
    const int r = r0 + threadIdx.x / TPR;
    const int rr = r < N ? r : N - 1;          // a row past the end repeats the last one
    float y[8];
    rotate_row8<D>(x, ((size_t)bh * N + rr) * D + 8 * c, signs, c, y);
#pragma unroll
    for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(y[t]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float b = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    atomicMax(amax_bits + bh, q_f2u(b));
  }
}

template <int D>
__global__ void __launch_bounds__(256) fa_rot_quant_kernel(const void* x, const signed char* signs,
                                                           uint8_t* out, const uint32_t* amax_bits, int N) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;
  const int bh = blockIdx.y;
  const int c = threadIdx.x % TPR;
  const float amax = q_u2f(amax_bits[bh]);
  const float mult = amax == 0.0f ? 1.0f : 448.0f / amax;
  for (int r0 = blockIdx.x * RPB; r0 < N; r0 += gridDim.x * RPB) {
    const int r = r0 + threadIdx.x / TPR;
    const int rr = r < N ? r : N - 1;
    float y[8];
    rotate_row8<D>(x, ((size_t)bh * N + rr) * D + 8 * c, signs, c, y);
    uint2 o;
    int pk0 = 0, pk1 = 0;
    float z[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) z[t] = fminf(fmaxf(y[t] * mult, -448.0f), 448.0f);
    pk0 = __builtin_amdgcn_cvt_pk_fp8_f32(z[0], z[1], pk0, false);
    pk0 = __builtin_amdgcn_cvt_pk_fp8_f32(z[2], z[3], pk0, true);
    pk1 = __builtin_amdgcn_cvt_pk_fp8_f32(z[4], z[5], pk1, false);
    pk1 = __builtin_amdgcn_cvt_pk_fp8_f32(z[6], z[7], pk1, true);
    o.x = (uint32_t)pk0;
    o.y = (uint32_t)pk1;
    if (r < N) *(uint2*)(out + ((size_t)bh * N + r) * D + 8 * c) = o;
  }
}

// amax (bit pattern, in place) -> descale = amax / 448 (or 1 for amax == 0),
// times `post` (1, or the exact power of two 1/d for a rotated Q)
__global__ void fa_descale_finalize_scaled(uint32_t* amax_bits_then_descale, int n, float post) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const float amax = q_u2f(amax_bits_then_descale[i]);
    const float ds = amax == 0.0f ? 1.0f : amax / 448.0f;
    amax_bits_then_descale[i] = q_f2u(ds * post);
  }
}

// ---------------------------------------------------------------------------
// Per-block FP8 ("Kernels and Memory in LLM Inference", section "Precision:
// FP8 with a real failure mode": a scale per block, so an outlier coarsens
// only its own block's grid). Blocks are 32 consecutive elements along the
// axis the product sums over (the layout of the OCP microscaling formats that
// gfx950's scaled MFMAs apply): 32 elements of a row for Q and K, 32 keys of
// a column for V. The scale is the power of two 2^e with the smallest e such
// that amax <= 448 * 2^e (so nothing saturates), stored as the E8M0 byte
// e + 127, e clamped to [-127, 127]; codes are e4m3 RNE of x * 2^-e. Every
// block is independent, so each kernel is one pass over its input.

// The block exponent from amax's bit pattern: amax = m 2^E with m in [1, 2)
// lies at or below 448 * 2^e = 1.75 * 2^(8 + e) for e = E - 8 when m <= 1.75
// (mantissa field <= 0x600000), else from e = E - 7. Zero and subnormal amax
// (below 2^-126) clamp to -127.
__device__ __forceinline__ int mx_block_exp(float amax) {
  const uint32_t b = q_f2u(amax);
  const int ef = (int)(b >> 23);
  if (ef == 0) return -127;
  const int e = ef - 135 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : e;
}

// 2^k as a float, for k in [-126, 127]
__device__ __forceinline__ float mx_exp2i(int k) { return q_u2f((uint32_t)(k + 127) << 23); }

__device__ __forceinline__ uint32_t mx_pack4(const float* v, float mult) {
  int pk = 0;
  pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * mult, v[1] * mult, pk, false);
  pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2] * mult, v[3] * mult, pk, true);
  return (uint32_t)pk;
}

// Row blocks (Q, K): thread t quantises elements [32t, 32t + 32) of the flat
// [B*H*N*d] input, writes their codes and scale byte t. `post` (1 or the power
// of two 1/d) multiplies every value first.
template <bool BF16>
__global__ void __launch_bounds__(256) fa_mx_rows_kernel(const void* x, uint8_t* out, uint8_t* scales,
                                                         long long nblocks, float post) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= nblocks) return;
  float v[32];
  load16<BF16>(x, (size_t)t * 32, v);
  load16<BF16>(x, (size_t)t * 32 + 16, v + 16);
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] *= post;
    m = fmaxf(m, fabsf(v[i]));
  }
  const int e = mx_block_exp(m);
  const float mult = mx_exp2i(-e);
  qu32x4 o0, o1;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    o0[w] = mx_pack4(v + 4 * w, mult);
    o1[w] = mx_pack4(v + 16 + 4 * w, mult);
  }
  qu32x4* dst = (qu32x4*)(out + (size_t)t * 32);
  dst[0] = o0;
  dst[1] = o1;
  scales[t] = (uint8_t)(e + 127);
}

// Row blocks after the randomised Hadamard rotation (bf16 input): the rows
// are rotated as in fa_rot_quant_kernel (D/8 lanes per row, 8 values each),
// scaled by `post`, and every 4 consecutive lanes (32 values) form one block.
template <int D>
__global__ void __launch_bounds__(256) fa_mx_rows_rot_kernel(const void* x, const signed char* signs,
                                                             uint8_t* out, uint8_t* scales, int N,
                                                             float post) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;
  const int bh = blockIdx.y;
  const int c = threadIdx.x % TPR;
  for (int r0 = blockIdx.x * RPB; r0 < N; r0 += gridDim.x * RPB) {
    const int r = r0 + threadIdx.x / TPR;
    const int rr = r < N ? r : N - 1;   // a row past the end repeats the last one
    float y[8];
    rotate_row8<D>(x, ((size_t)bh * N + rr) * D + 8 * c, signs, c, y);
    float m = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      y[t] *= post;
      m = fmaxf(m, fabsf(y[t]));
    }
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    const int e = mx_block_exp(m);
    const float mult = mx_exp2i(-e);
    uint2 o;
    o.x = mx_pack4(y, mult);
    o.y = mx_pack4(y + 4, mult);
    if (r < N) {
      *(uint2*)(out + ((size_t)bh * N + r) * D + 8 * c) = o;
      if ((c & 3) == 0) scales[((size_t)bh * N + r) * (D / 32) + c / 4] = (uint8_t)(e + 127);
    }
  }
}

// Key blocks (V): thread t takes 4 consecutive columns of one 32-key block of
// one head: items = B*H * ceil(N/32) * D/4; two passes over the block's rows
// (amax, then codes), one dword of codes per key and one of scale bytes.
template <bool BF16, int D>
__global__ void __launch_bounds__(256) fa_mx_keys_kernel(const void* x, uint8_t* out, uint8_t* scales,
                                                         int N, int nkb, long long items) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= items) return;
  const int cg = (int)(t % (D / 4));
  const long long rb = t / (D / 4);
  const int kb = (int)(rb % nkb);
  const long long bh = rb / nkb;
  const int k0 = 32 * kb;
  const int k1 = k0 + 32 < N ? k0 + 32 : N;
  auto load4 = [&](int k, float* v) {
    const size_t e0 = ((size_t)bh * N + k) * D + 4 * cg;
    if constexpr (BF16) {
      const uint2 w = *(const uint2*)((const unsigned short*)x + e0);
      v[0] = q_u2f(w.x << 16);
      v[1] = q_u2f(w.x & 0xffff0000u);
      v[2] = q_u2f(w.y << 16);
      v[3] = q_u2f(w.y & 0xffff0000u);
    } else {
      const qu32x4 w = *(const qu32x4*)((const float*)x + e0);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = q_u2f(w[i]);
    }
  };
  float m[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k = k0; k < k1; ++k) {
    float v[4];
    load4(k, v);
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = fmaxf(m[i], fabsf(v[i]));
  }
  int e[4];
  float mult[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e[i] = mx_block_exp(m[i]);
    mult[i] = mx_exp2i(-e[i]);
  }
  for (int k = k0; k < k1; ++k) {
    float v[4];
    load4(k, v);
    int pk = 0;
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * mult[0], v[1] * mult[1], pk, false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2] * mult[2], v[3] * mult[3], pk, true);
    *(uint32_t*)(out + ((size_t)bh * N + k) * D + 4 * cg) = (uint32_t)pk;
  }
  const uint32_t sc = (uint32_t)(e[0] + 127) | ((uint32_t)(e[1] + 127) << 8) |
                      ((uint32_t)(e[2] + 127) << 16) | ((uint32_t)(e[3] + 127) << 24);
  *(uint32_t*)(scales + ((size_t)bh * nkb + kb) * D + 4 * cg) = sc;
}

// amax (bit pattern, in place) -> descale = amax / 448, or 1 for amax == 0
__global__ void fa_descale_finalize(uint32_t* amax_bits_then_descale, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const float amax = q_u2f(amax_bits_then_descale[i]);
    const float ds = amax == 0.0f ? 1.0f : amax / 448.0f;
    amax_bits_then_descale[i] = q_f2u(ds);
  }
}

}  // namespace fa
