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
  // four strides per trip: every load of the trip is in flight before the
  // first max, and four independent max chains
  constexpr int U = 4;
  const long long stride = (long long)gridDim.x * blockDim.x;
  float mu[U] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (long long t0 = (long long)blockIdx.x * blockDim.x + threadIdx.x; t0 < n16; t0 += U * stride) {
    float v[U][16];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long t = t0 + u * stride;
      if (t < n16) {
        load16<BF16>(x, head0 + (size_t)t * 16, v[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[u][i] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) mu[u] = fmaxf(mu[u], fabsf(v[u][i]));
  }
  float m = fmaxf(fmaxf(mu[0], mu[1]), fmaxf(mu[2], mu[3]));
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
// D/32 consecutive lanes (a quarter or half of a DPP quad) holding 32
// consecutive elements each: butterflies of stride 1..16 inside a lane,
// strides 32 and 64 between the lanes of the quad with DPP quad permutes (no
// LDS traffic). Every butterfly is one v_fma_f64 with a weight of +-1, exact.

// Sign masks of lane c, one per bf16 pair: word j has bit 15 set when
// element 32c + 2j is negated and bit 31 when element 32c + 2j + 1 is, so one
// XOR with the loaded pair applies both signs.
struct RotSigns {
  uint32_t w[16];
};
__device__ __forceinline__ RotSigns rot_sign_mask(const signed char* signs, int c) {
  RotSigns m;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    m.w[j] = (signs[32 * c + 2 * j] < 0 ? 0x8000u : 0u) | (signs[32 * c + 2 * j + 1] < 0 ? 0x80000000u : 0u);
  return m;
}

// v from the lane that differs in bit M of its quad position (M = 1 or 2)
template <int M>
__device__ __forceinline__ double quad_xor(double v) {
  static_assert(M == 1 || M == 2, "quad permutes only");
  constexpr int kCtrl = M == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, kCtrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), kCtrl, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
}

// y[t] = element 32c + t of the rotated row whose bf16 elements 32c .. 32c+31
// start at element e0 of x (lane c of the row's D/32 lanes)
template <int D>
__device__ __forceinline__ void rotate_row32(const void* x, size_t e0, const RotSigns& neg, int c, float* y) {
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  const qu32x4* src = (const qu32x4*)((const unsigned short*)x + e0);
  double v[32];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const qu32x4 w = src[h];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = 8 * h + 2 * k;
      const uint32_t p = w[k] ^ neg.w[t / 2];
      v[t] = (double)q_u2f(p << 16);
      v[t + 1] = (double)q_u2f(p & 0xffff0000u);
    }
  }
#pragma unroll
  for (int h = 1; h < 32; h <<= 1)
#pragma unroll
    for (int t = 0; t < 32; ++t)
      if ((t & h) == 0) {
        const double a = v[t], b = v[t + h];
        v[t] = a + b;
        v[t + h] = a - b;
      }
  // the lane with the higher element index keeps lower - upper
  {
    const double w1 = (c & 1) ? -1.0 : 1.0;
#pragma unroll
    for (int t = 0; t < 32; ++t) v[t] = __builtin_fma(v[t], w1, quad_xor<1>(v[t]));
  }
  if constexpr (D == 128) {
    const double w2 = (c & 2) ? -1.0 : 1.0;
#pragma unroll
    for (int t = 0; t < 32; ++t) v[t] = __builtin_fma(v[t], w2, quad_xor<2>(v[t]));
  }
#pragma unroll
  for (int t = 0; t < 32; ++t) y[t] = (float)v[t];
}

// grid = (blocks per head, B*H); rows of D bf16, D/32 lanes per row
template <int D>
__global__ void __launch_bounds__(256) fa_rot_amax_kernel(const void* x, const signed char* signs,
                                                          uint32_t* amax_bits, int N) {
  constexpr int TPR = D / 32, RPB = 256 / TPR;
  const int bh = blockIdx.y;
  const int c = threadIdx.x % TPR;
  const RotSigns neg = rot_sign_mask(signs, c);
  float m = 0.0f;
  for (int r0 = blockIdx.x * RPB; r0 < N; r0 += gridDim.x * RPB) {
    const int r = r0 + threadIdx.x / TPR;
    const int rr = r < N ? r : N - 1;          // a row past the end repeats the last one
    float y[32];
    rotate_row32<D>(x, ((size_t)bh * N + rr) * D + 32 * c, neg, c, y);
#pragma unroll
    for (int t = 0; t < 32; ++t) m = fmaxf(m, fabsf(y[t]));
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
  constexpr int TPR = D / 32, RPB = 256 / TPR;
  const int bh = blockIdx.y;
  const int c = threadIdx.x % TPR;
  const RotSigns neg = rot_sign_mask(signs, c);
  const float amax = q_u2f(amax_bits[bh]);
  const float mult = amax == 0.0f ? 1.0f : 448.0f / amax;
  for (int r0 = blockIdx.x * RPB; r0 < N; r0 += gridDim.x * RPB) {
    const int r = r0 + threadIdx.x / TPR;
    const int rr = r < N ? r : N - 1;
    float y[32];
    rotate_row32<D>(x, ((size_t)bh * N + rr) * D + 32 * c, neg, c, y);
    qu32x4 o[2];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      float z[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) z[t] = fminf(fmaxf(y[4 * w + t] * mult, -448.0f), 448.0f);
      int pk = 0;
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(z[0], z[1], pk, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(z[2], z[3], pk, true);
      o[w >> 2][w & 3] = (uint32_t)pk;
    }
    if (r < N) {
      qu32x4* dst = (qu32x4*)(out + ((size_t)bh * N + r) * D + 32 * c);
      dst[0] = o[0];
      dst[1] = o[1];
    }
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
  constexpr int TPR = D / 32, RPB = 256 / TPR;
  const int bh = blockIdx.y;
  const int c = threadIdx.x % TPR;
  const RotSigns neg = rot_sign_mask(signs, c);
  for (int r0 = blockIdx.x * RPB; r0 < N; r0 += gridDim.x * RPB) {
    const int r = r0 + threadIdx.x / TPR;
    const int rr = r < N ? r : N - 1;   // a row past the end repeats the last one
    float y[32];
    rotate_row32<D>(x, ((size_t)bh * N + rr) * D + 32 * c, neg, c, y);
    // the lane's 32 values are exactly one block
    float m = 0.0f;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      y[t] *= post;
      m = fmaxf(m, fabsf(y[t]));
    }
    const int e = mx_block_exp(m);
    const float mult = mx_exp2i(-e);
    qu32x4 o[2];
#pragma unroll
    for (int w = 0; w < 8; ++w) o[w >> 2][w & 3] = mx_pack4(y + 4 * w, mult);
    if (r < N) {
      qu32x4* dst = (qu32x4*)(out + ((size_t)bh * N + r) * D + 32 * c);
      dst[0] = o[0];
      dst[1] = o[1];
      scales[((size_t)bh * N + r) * (D / 32) + c] = (uint8_t)(e + 127);
    }
  }
}

// Key blocks (V): thread t takes 4 consecutive columns of one 32-key block of
// one head: items = B*H * ceil(N/32) * D/4; one dword of codes per key and one
// of scale bytes. A whole bf16 block is read once into registers (amax, then
// codes from the registers); fp32 input and a ragged last block take two
// passes over the block's rows.
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
  auto store4 = [&](int k, const float* v, const float* mult) {
    int pk = 0;
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * mult[0], v[1] * mult[1], pk, false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2] * mult[2], v[3] * mult[3], pk, true);
    *(uint32_t*)(out + ((size_t)bh * N + k) * D + 4 * cg) = (uint32_t)pk;
  };
  float m[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int e[4];
  float mult[4];
  if (BF16 && k1 - k0 == 32) {
    // the block's raw bf16 pairs stay in registers (64 of them)
    uint2 w[32];
    auto unpack = [](uint2 p, float* v) {
      v[0] = q_u2f(p.x << 16);
      v[1] = q_u2f(p.x & 0xffff0000u);
      v[2] = q_u2f(p.y << 16);
      v[3] = q_u2f(p.y & 0xffff0000u);
    };
#pragma unroll
    for (int k = 0; k < 32; ++k)
      w[k] = *(const uint2*)((const unsigned short*)x + ((size_t)bh * N + k0 + k) * D + 4 * cg);
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      float v[4];
      unpack(w[k], v);
#pragma unroll
      for (int i = 0; i < 4; ++i) m[i] = fmaxf(m[i], fabsf(v[i]));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[i] = mx_block_exp(m[i]);
      mult[i] = mx_exp2i(-e[i]);
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      float v[4];
      unpack(w[k], v);
      store4(k0 + k, v, mult);
    }
  } else {
    for (int k = k0; k < k1; ++k) {
      float v[4];
      load4(k, v);
#pragma unroll
      for (int i = 0; i < 4; ++i) m[i] = fmaxf(m[i], fabsf(v[i]));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[i] = mx_block_exp(m[i]);
      mult[i] = mx_exp2i(-e[i]);
    }
    for (int k = k0; k < k1; ++k) {
      float v[4];
      load4(k, v);
      store4(k, v, mult);
    }
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
