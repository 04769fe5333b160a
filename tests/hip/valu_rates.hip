// Test helper (not part of libfa): issue cost of the VALU operations the
// softmax is made of, on one SIMD shared by two waves. Every launch has 256
// workgroups of 512 threads (8 waves, two per SIMD); waves 0-3 run role A,
// waves 4-7 role B, each 64 dependent-chain operations per iteration on 16
// independent values; thread t of workgroup b writes out[512 b + t] only.
//   role 0: idle;  1: v_fma_f32;  2: v_exp_f32;
//   role 3: exp2 from FMAs (Cody-Waite split n = rint(x), f = x - n, a
//           degree-4 polynomial in f, ldexp by n): the "exp2 on FMA units"
//           of FlashAttention-4.
#include <hip/hip_runtime.h>

template <int ROLE>
__device__ __forceinline__ float role(int iters, float a) {
  float x[16];
  for (int i = 0; i < 16; ++i) x[i] = -(float)(threadIdx.x & 7) * 0.1f - 0.05f * i;
  if constexpr (ROLE == 0) return a;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 64; ++k) {
      float& y = x[k & 15];
      if constexpr (ROLE == 1) {
        y = __builtin_fmaf(y, a, -0.5f);
      } else if constexpr (ROLE == 2) {
        y = __builtin_amdgcn_exp2f(y) - 1.0f;
      } else {
        const float n = __builtin_rintf(y);
        const float f = y - n;
        // Taylor coefficients of 2^f: (ln 2)^k / k!
        float p = __builtin_fmaf(f, 0.0096181291f, 0.0555041087f);
        p = __builtin_fmaf(p, f, 0.2402265070f);
        p = __builtin_fmaf(p, f, 0.6931471806f);
        p = __builtin_fmaf(p, f, 1.0f);
        y = __builtin_amdgcn_ldexpf(p, (int)n) - 1.0f;
      }
    }
  }
  float s = 0.0f;
  for (int i = 0; i < 16; ++i) s += x[i];
  return s;
}

template <int RA, int RB>
__global__ void __launch_bounds__(512) valu_pair(float* out, float a, int iters) {
  const int w = threadIdx.x >> 6;
  const float s = w < 4 ? role<RA>(iters, a) : role<RB>(iters, a);
  out[blockIdx.x * 512 + threadIdx.x] = s;
}

// relative error of the FMA exp2 against v_exp_f32 at 65536 points of [-30, 0]
__global__ void poly_error(float* out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const float y = -30.0f * (float)i / 65536.0f;
  const float n = __builtin_rintf(y);
  const float f = y - n;
  float p = __builtin_fmaf(f, 0.0096181291f, 0.0555041087f);
  p = __builtin_fmaf(p, f, 0.2402265070f);
  p = __builtin_fmaf(p, f, 0.6931471806f);
  p = __builtin_fmaf(p, f, 1.0f);
  const float e = __builtin_amdgcn_exp2f(y);
  out[i] = fabsf(__builtin_amdgcn_ldexpf(p, (int)n) - e) / e;
}

// pair = 10 * role A + role B. Mean microseconds per launch over 5 launches
// after a warm-up in *us; 0 on success, -1 on a HIP error.
extern "C" int valu_pair_run(int pair, int iters, float* us) {
  float* out = nullptr;
  if (hipMalloc(&out, 256 * 512 * sizeof(float)) != hipSuccess) return -1;
  auto launch = [&]() {
    const dim3 g(256), b(512);
    switch (pair) {
      case 10: hipLaunchKernelGGL((valu_pair<1, 0>), g, b, 0, 0, out, 0.9999f, iters); break;
      case 20: hipLaunchKernelGGL((valu_pair<2, 0>), g, b, 0, 0, out, 0.9999f, iters); break;
      case 30: hipLaunchKernelGGL((valu_pair<3, 0>), g, b, 0, 0, out, 0.9999f, iters); break;
      case 11: hipLaunchKernelGGL((valu_pair<1, 1>), g, b, 0, 0, out, 0.9999f, iters); break;
      case 22: hipLaunchKernelGGL((valu_pair<2, 2>), g, b, 0, 0, out, 0.9999f, iters); break;
      case 12: hipLaunchKernelGGL((valu_pair<1, 2>), g, b, 0, 0, out, 0.9999f, iters); break;
      case 23: hipLaunchKernelGGL((valu_pair<2, 3>), g, b, 0, 0, out, 0.9999f, iters); break;
      default: break;
    }
  };
  int rc = 0;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) rc = -1;
  if (rc == 0) {
    launch();
    (void)hipEventRecord(e0, 0);
    for (int r = 0; r < 5; ++r) launch();
    (void)hipEventRecord(e1, 0);
    float ms = 0.0f;
    if (hipGetLastError() != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
      rc = -1;
    else
      *us = ms / 5 * 1000.0f;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
  }
  (void)hipFree(out);
  return rc;
}

// max relative error of the FMA exp2 over [-30, 0] in *err; 0 on success
extern "C" int poly_exp2_error(float* err) {
  float* out = nullptr;
  if (hipMalloc(&out, 65536 * sizeof(float)) != hipSuccess) return -1;
  hipLaunchKernelGGL(poly_error, dim3(256), dim3(256), 0, 0, out);
  static float h[65536];
  int rc = hipMemcpy(h, out, sizeof(h), hipMemcpyDeviceToHost) == hipSuccess ? 0 : -1;
  float m = 0.0f;
  for (int i = 0; i < 65536; ++i) m = h[i] > m ? h[i] : m;
  *err = m;
  (void)hipFree(out);
  return rc;
}
