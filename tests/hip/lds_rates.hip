// Test helper (not part of libfa): LDS read throughput of one workgroup for a
// given per-lane address pattern. Every wave of the workgroup runs the same
// pattern: per trip 16 independent reads at offs[lane] + 2048 u (u = 0..15,
// a multiple of the 256-byte bank period, so every read sees the same banks),
// as ds_read_b128 (kind 0) or ds_read_b64_tr_b16 (kind 1). Reports cycles per
// read per wave. Every address stays below 64 KB; the host checks offs.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;

template <int KIND>
__global__ void __launch_bounds__(1024) lds_rate_kernel(const uint32_t* offs, uint32_t* sink, long long* cycles,
                                                        int trips) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[65536];
  const int tid = threadIdx.x;
  for (int i = tid; i < 65536 / 4; i += blockDim.x) ((uint32_t*)smem)[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  uint32_t off = offs[tid & 63];
  uint32_t acc = 0;
  const long long t0 = clock64();
  for (int it = 0; it < trips; ++it) {
    asm volatile("" : "+v"(off));   // opaque address: the reads stay in the loop
    uint32_t w[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const unsigned char* src = smem + off + 2048 * u;
      if constexpr (KIND == 0) {
        const u32x4_t x = *(const u32x4_t*)src;
        w[u] = x[0] + 5u * x[1] + 7u * x[2] + x[3];
      } else {
        const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)src);
        w[u] = (uint32_t)(unsigned short)v[0] + 3u * (uint32_t)(unsigned short)v[1] +
               5u * (uint32_t)(unsigned short)v[2] + (uint32_t)(unsigned short)v[3];
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) acc = acc * 3u + w[u];
  }
  __syncthreads();
  const long long t1 = clock64();
  sink[tid] = acc;
  if (tid == 0) cycles[0] = t1 - t0;
}

// kind 0: ds_read_b128, 1: ds_read_b64_tr_b16; threads = 64 * waves (<= 1024);
// offs: 64 offsets (16-byte aligned for kind 0, 8-byte for kind 1) with
// offs + 30720 + 16 <= 65536; sink: `threads` words; cycles: 1 value.
extern "C" int lds_rate_run(int kind, const uint32_t* offs, uint32_t* sink, long long* cycles, int trips,
                            int threads) {
  if (threads < 64 || threads > 1024 || threads % 64 != 0) return -1;
  if (kind == 0)
    hipLaunchKernelGGL(lds_rate_kernel<0>, dim3(1), dim3(threads), 0, 0, offs, sink, cycles, trips);
  else
    hipLaunchKernelGGL(lds_rate_kernel<1>, dim3(1), dim3(threads), 0, 0, offs, sink, cycles, trips);
  return (int)hipDeviceSynchronize();
}
