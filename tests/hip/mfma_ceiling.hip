// Test helper (not part of libfa): the sustained rate of the 32x32 bf16 and fp8
// MFMAs the attention kernel uses, with the operand data held constant or
// drawn at random. MI355X lowers its clock when the matrix cores switch many
// bits, so the rate reachable on real data sits below the published peak; this
// measures how far. The loop has the shape of one key tile of the attention
// kernel's products: a chain of MFMAs on one accumulator (the scores), then
// MFMAs into four others (the output), with nothing else in between. A second
// kernel runs the same random-data flop stream on the 16x16 MFMA shapes beside
// the 32x32 ones, with and without exp/fma work interleaved, to show which
// shape an attention kernel (whose softmax shares the issue slots) should use.
//
// Every launch: `blocks` workgroups of 256 threads (4 waves), three waves per
// SIMD; thread t of workgroup b writes one float to out[256 b + t], nothing
// else touches memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// integer hash (xor-shift-multiply mixer) -> pseudo-random 32-bit words
__device__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// roughly N(0, 1): centred sum of the four bytes of a hash
__device__ float normalish(uint32_t x) {
  const uint32_t h = mix32(x);
  const float s = (float)(h & 255u) + (float)((h >> 8) & 255u) + (float)((h >> 16) & 255u) +
                  (float)(h >> 24);
  return (s - 510.0f) / 147.8f;
}

// four random e4m3fn bytes, with the two NaN codes (0x7f, 0xff) moved to 0x7e / 0xfe
__device__ int fp8x4(uint32_t x) {
  uint32_t h = mix32(x);
  for (int b = 0; b < 4; ++b)
    if (((h >> (8 * b)) & 0x7fu) == 0x7fu) h ^= 1u << (8 * b);
  return (int)h;
}

template <bool RANDOM>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
ceiling_bf16(float* out, int iters) {
  const uint32_t tid = blockIdx.x * 256u + threadIdx.x;
  bf16x8 a[8], b[8];
  for (int k = 0; k < 8; ++k)
    for (int i = 0; i < 8; ++i) {
      a[k][i] = (__bf16)(RANDOM ? normalish(tid * 131u + 8u * k + i) : 0.5f);
      b[k][i] = (__bf16)(RANDOM ? normalish((tid * 131u + 8u * k + i) ^ 0x9e3779b9u) : 0.25f);
    }
  f32x16 o[4];
  for (int m = 0; m < 4; ++m) o[m] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) asm volatile("" : "+v"(a[k]));   // a fresh operand every tile
    f32x16 s = f32x16{};
#pragma unroll
    for (int k = 0; k < 8; ++k) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[k], s, 0, 0, 0);
    bf16x8 p0, p1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p0[i] = (__bf16)(s[i] * 0.05f);
      p1[i] = (__bf16)(s[8 + i] * 0.05f);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      o[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2 * m], p0, o[m], 0, 0, 0);
      o[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2 * m + 1], p1, o[m], 0, 0, 0);
    }
  }
  float r = 0.0f;
  for (int m = 0; m < 4; ++m)
    for (int i = 0; i < 16; ++i) r += o[m][i];
  out[tid] = r;
}

template <bool RANDOM>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
ceiling_fp8(float* out, int iters) {
  const uint32_t tid = blockIdx.x * 256u + threadIdx.x;
  i32x8 a[2], b[2];
  for (int k = 0; k < 2; ++k)
    for (int i = 0; i < 8; ++i) {
      a[k][i] = RANDOM ? fp8x4(tid * 131u + 8u * k + i) : 0x38383838;   // 1.0
      b[k][i] = RANDOM ? fp8x4((tid * 131u + 8u * k + i) ^ 0x9e3779b9u) : 0x30303030;   // 0.5
    }
  f32x16 o[4];
  for (int m = 0; m < 4; ++m) o[m] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 2; ++k) asm volatile("" : "+v"(a[k]));
    // two 32-key score blocks of two MFMAs each, then four output MFMAs
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[k], b[k], s0, 0, 0, 0, 127, 0, 127);
      s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[k], a[k], s1, 0, 0, 0, 127, 0, 127);
    }
    i32x8 p;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      int v = 0;
      v = __builtin_amdgcn_cvt_pk_fp8_f32(s0[2 * w] * 0.01f, s0[2 * w + 1] * 0.01f, v, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(s1[2 * w] * 0.01f, s1[2 * w + 1] * 0.01f, v, true);
      p[w] = v;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
      o[m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[m & 1], p, o[m], 0, 0, 0, 127, 0, 127);
  }
  float r = 0.0f;
  for (int m = 0; m < 4; ++m)
    for (int i = 0; i < 16; ++i) r += o[m][i];
  out[tid] = r;
}

// The same flop stream on the 32x32 and on the 16x16 MFMA shapes, optionally
// with softmax-like VALU work (an exp2 of an fma, on eight independent chains)
// issued between the MFMAs at a fixed number per flop. Per wave and iteration:
// bf16 8 x 32x32x16 or 16 x 16x16x32 (262144 flop), fp8 8 x 32x32x64 or
// 16 x 16x16x128 (1048576 flop); VALU pairs: 4 (bf16) or 8 (fp8) per 32x32
// MFMA, half that per 16x16 MFMA, when VALU is set.
template <bool FP8, bool SHAPE16, bool VALU>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
shape_mix(float* out, int iters) {
  const uint32_t tid = blockIdx.x * 256u + threadIdx.x;
  constexpr int NV = VALU ? (FP8 ? 8 : 4) : 0;
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = normalish(tid * 7u + i) * 0.01f;
  float r = 0.0f;
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type opnd;
  // four fp8 operand pairs (8 VGPRs each) keep the wave within the 168 VGPRs of
  // three waves per SIMD; eight bf16 pairs (4 each) do too
  constexpr int NQ = FP8 ? 4 : 8;
  opnd a[NQ], b[NQ];
  for (int q = 0; q < NQ; ++q)
    for (int i = 0; i < 8; ++i) {
      const uint32_t h = tid * 131u + 8u * q + i;
      if constexpr (FP8) {
        a[q][i] = fp8x4(h);
        b[q][i] = fp8x4(h ^ 0x9e3779b9u);
      } else {
        a[q][i] = (__bf16)normalish(h);
        b[q][i] = (__bf16)normalish(h ^ 0x9e3779b9u);
      }
    }
  if constexpr (!SHAPE16) {
    f32x16 o[4];
    for (int m = 0; m < 4; ++m) o[m] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) asm volatile("" : "+v"(a[q]));
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if constexpr (FP8)
          o[q & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[q % NQ], b[q % NQ], o[q & 3], 0, 0, 0, 127, 0, 127);
        else
          o[q & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[q % NQ], b[q % NQ], o[q & 3], 0, 0, 0);
#pragma unroll
        for (int v = 0; v < NV; ++v) x[v & 7] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[v & 7], 0.999f, -0.001f));
      }
    }
    for (int m = 0; m < 4; ++m)
      for (int i = 0; i < 16; ++i) r += o[m][i];
  } else {
    f32x4 o[8];
    for (int m = 0; m < 8; ++m) o[m] = f32x4{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) asm volatile("" : "+v"(a[q]));
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if constexpr (FP8) {
          o[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[q % NQ], b[q % NQ], o[q], 0, 0, 0, 127, 0, 127);
          o[(q + 4) & 7] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[q % NQ], a[q % NQ], o[(q + 4) & 7], 0, 0, 0, 127, 0, 127);
        } else {
          o[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q % NQ], b[q % NQ], o[q], 0, 0, 0);
          o[(q + 4) & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[q % NQ], a[q % NQ], o[(q + 4) & 7], 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) x[v & 7] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[v & 7], 0.999f, -0.001f));
      }
    }
    for (int m = 0; m < 8; ++m)
      for (int i = 0; i < 4; ++i) r += o[m][i];
  }
  for (int i = 0; i < 8; ++i) r += x[i];
  out[tid] = r;
}

// kind 0 = bf16 (16 MFMAs of 32768 flop per wave per iteration), 1 = fp8
// (8 MFMAs of 131072 flop); kinds 2..9 = shape_mix with 2 + 4 fp8 + 2 shape16
// + valu (random operands whatever `random` says). Times `reps` launches after one warm-up launch and
// returns the mean milliseconds per launch in *ms; 0 on success, -1 on a HIP
// error.
extern "C" int mfma_ceiling_run(int kind, int random, int blocks, int iters, int reps, float* ms) {
  if (kind < 0 || kind > 9 || blocks < 1 || iters < 1 || reps < 1 || !ms) return -1;
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)) != hipSuccess) return -1;
  auto launch = [&]() {
    const dim3 g((unsigned)blocks), b(256);
    switch (kind) {
      case 2: hipLaunchKernelGGL((shape_mix<false, false, false>), g, b, 0, 0, out, iters); return;
      case 3: hipLaunchKernelGGL((shape_mix<false, false, true>), g, b, 0, 0, out, iters); return;
      case 4: hipLaunchKernelGGL((shape_mix<false, true, false>), g, b, 0, 0, out, iters); return;
      case 5: hipLaunchKernelGGL((shape_mix<false, true, true>), g, b, 0, 0, out, iters); return;
      case 6: hipLaunchKernelGGL((shape_mix<true, false, false>), g, b, 0, 0, out, iters); return;
      case 7: hipLaunchKernelGGL((shape_mix<true, false, true>), g, b, 0, 0, out, iters); return;
      case 8: hipLaunchKernelGGL((shape_mix<true, true, false>), g, b, 0, 0, out, iters); return;
      case 9: hipLaunchKernelGGL((shape_mix<true, true, true>), g, b, 0, 0, out, iters); return;
      default: break;
    }
    if (kind == 0) {
      if (random) hipLaunchKernelGGL(ceiling_bf16<true>, g, b, 0, 0, out, iters);
      else hipLaunchKernelGGL(ceiling_bf16<false>, g, b, 0, 0, out, iters);
    } else {
      if (random) hipLaunchKernelGGL(ceiling_fp8<true>, g, b, 0, 0, out, iters);
      else hipLaunchKernelGGL(ceiling_fp8<false>, g, b, 0, 0, out, iters);
    }
  };
  hipEvent_t e0, e1;
  int rc = 0;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) rc = -1;
  if (rc == 0) {
    launch();
    if (hipEventRecord(e0, 0) != hipSuccess) rc = -1;
    for (int r = 0; r < reps && rc == 0; ++r) launch();
    if (hipGetLastError() != hipSuccess || hipEventRecord(e1, 0) != hipSuccess ||
        hipEventSynchronize(e1) != hipSuccess)
      rc = -1;
    float t = 0.0f;
    if (rc == 0 && hipEventElapsedTime(&t, e0, e1) == hipSuccess) *ms = t / reps;
    else rc = -1;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
  }
  (void)hipFree(out);
  return rc;
}
