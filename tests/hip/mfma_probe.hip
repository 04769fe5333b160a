// Test helper (not part of libfa): one-wave kernels that run a single MFMA on
// operands given per lane and return every accumulator register, so a test
// can check on the host the lane layouts the attention kernel relies on and
// the accumulation precision of the fp8 MFMA. Every launch is one wave of 64
// lanes reading 64*K inputs and writing 64*16 outputs.
#include <hip/hip_runtime.h>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__global__ void probe_f32_kernel(const float* a, const float* b, float* c) {
  const int l = threadIdx.x;
  f32x16 acc = {};
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[l], b[l], acc, 0, 0, 0);
  for (int r = 0; r < 16; ++r) c[l * 16 + r] = acc[r];
}

__global__ void probe_bf16_kernel(const float* a, const float* b, float* c) {
  const int l = threadIdx.x;
  f32x16 acc = {};
  bf16x8 av, bv;
  for (int s = 0; s < 8; ++s) {
    av[s] = (__bf16)a[l * 8 + s];
    bv[s] = (__bf16)b[l * 8 + s];
  }
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
  for (int r = 0; r < 16; ++r) c[l * 16 + r] = acc[r];
}

__global__ void probe_fp8_kernel(const int* a, const int* b, float* c) {
  const int l = threadIdx.x;
  f32x16 acc = {};
  i32x8 av, bv;
  for (int s = 0; s < 8; ++s) {
    av[s] = a[l * 8 + s];
    bv[s] = b[l * 8 + s];
  }
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
  for (int r = 0; r < 16; ++r) c[l * 16 + r] = acc[r];
}

// The scaled fp8 MFMA with a 32-bit scale register per lane for each operand;
// OPA / OPB pick the byte of that register the instruction uses (E8M0:
// 2^(byte - 127)).
template <int OPA, int OPB>
__global__ void probe_fp8_scaled_kernel(const int* a, const int* b, const int* sa, const int* sb,
                                        float* c) {
  const int l = threadIdx.x;
  f32x16 acc = {};
  i32x8 av, bv;
  for (int s = 0; s < 8; ++s) {
    av[s] = a[l * 8 + s];
    bv[s] = b[l * 8 + s];
  }
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, OPA, sa[l], OPB, sb[l]);
  for (int r = 0; r < 16; ++r) c[l * 16 + r] = acc[r];
}

// variant 0: bytes (0, 0); 1: (2, 1); 2: (3, 3). a, b: 64 x 32 codes; sa, sb:
// 64 scale registers; c: 64 x 16 floats.
extern "C" int probe_mfma_scaled(int variant, const void* a, const void* b, const void* sa,
                                 const void* sb, float* c) {
  const int *pa = (const int*)a, *pb = (const int*)b, *psa = (const int*)sa, *psb = (const int*)sb;
  if (variant == 0)
    hipLaunchKernelGGL((probe_fp8_scaled_kernel<0, 0>), dim3(1), dim3(64), 0, 0, pa, pb, psa, psb, c);
  else if (variant == 1)
    hipLaunchKernelGGL((probe_fp8_scaled_kernel<2, 1>), dim3(1), dim3(64), 0, 0, pa, pb, psa, psb, c);
  else
    hipLaunchKernelGGL((probe_fp8_scaled_kernel<3, 3>), dim3(1), dim3(64), 0, 0, pa, pb, psa, psb, c);
  return (int)hipDeviceSynchronize();
}

extern "C" int probe_mfma(int kind, const void* a, const void* b, float* c) {
  if (kind == 0)
    hipLaunchKernelGGL(probe_f32_kernel, dim3(1), dim3(64), 0, 0, (const float*)a, (const float*)b, c);
  else if (kind == 1)
    hipLaunchKernelGGL(probe_bf16_kernel, dim3(1), dim3(64), 0, 0, (const float*)a, (const float*)b, c);
  else
    hipLaunchKernelGGL(probe_fp8_kernel, dim3(1), dim3(64), 0, 0, (const int*)a, (const int*)b, c);
  return (int)hipDeviceSynchronize();
}
