// C ABI of libfa.so: argument validation, choice of kernel instantiation, and
// launch on the caller's stream. The declarations and the contract of every
// entry point are in include/fa.h.
#include <climits>
#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_fwd_kernel.hpp"
#include "fa_quant_kernel.hpp"

namespace {

// Tile shapes: 4 waves x 32 query rows per workgroup; key tile 64 (bf16, fp8)
// or 32 (fp32); registers bounded so two workgroups share a CU (2 waves per
// SIMD): a single wave per SIMD cannot keep the MFMA pipe busy.
constexpr int kWaves = 4;
constexpr int kWavesPerSimd = 2;

// Head dim 128, bf16 and fp8: global -> LDS by DMA, V^T read with the LDS
// transpose reads (the shapes the DiT benchmark runs). bf16: key tile 32,
// three stages, three waves per SIMD; fp8: key tile 64, two stages, three
// waves per SIMD.
template <int DT>
int launch_fwd_dma(fa::FwdArgs a, bool causal, hipStream_t stream) {
  constexpr int BN = DT == fa::kBF16 ? 32 : 64;
  constexpr int NSTAGE = DT == fa::kBF16 ? 3 : 2;
  constexpr int LOOK = 2, WPE = 3;
  const dim3 grid((unsigned)((long long)a.BH * a.n_qtiles));
  const dim3 block(64 * kWaves);
  if (causal)
    hipLaunchKernelGGL((fa::fa_fwd_dma_kernel<DT, BN, kWaves, true, LOOK, WPE, NSTAGE>), grid, block, 0,
                       stream, a);
  else
    hipLaunchKernelGGL((fa::fa_fwd_dma_kernel<DT, BN, kWaves, false, LOOK, WPE, NSTAGE>), grid, block, 0,
                       stream, a);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <int DT, int D, int BN>
int launch_fwd(const fa::FwdArgs& a, bool causal, hipStream_t stream) {
  using C = fa::Cfg<DT, D, BN, kWaves>;
  const dim3 grid((unsigned)((long long)a.BH * a.n_qtiles));
  const dim3 block(C::NT);
  if (causal)
    hipLaunchKernelGGL((fa::fa_fwd_kernel<DT, D, BN, kWaves, true, kWavesPerSimd>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fa::fa_fwd_kernel<DT, D, BN, kWaves, false, kWavesPerSimd>), grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: B, H or N is negative or the problem is too large";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: unknown dtype";
    case FA_ERR_HEAD_DIM: return "FA_ERR_HEAD_DIM: head dim must be 64 or 128";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite";
    case FA_ERR_DESCALES: return "FA_ERR_DESCALES: FP8 needs a descale array";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: tensor pointers must be 16-byte aligned";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime rejected a launch";
    default: return "unknown fa status";
  }
}

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int d, int causal, float scale, int dtype,
                      const float* descales, hipStream_t stream) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP8_E4M3)
    return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (dtype == FA_DTYPE_FP8_E4M3 && descales == nullptr) return FA_ERR_DESCALES;
  const long long BH = (long long)B * H;
  if (BH == 0 || N == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_ALIGN;
  const int BM = 32 * kWaves;
  const long long n_qtiles = ((long long)N + BM - 1) / BM;
  if (BH > INT_MAX || BH * n_qtiles > INT_MAX) return FA_ERR_SHAPE;
  // one head of Q, K or V is addressed with 32-bit buffer offsets
  const long long es = dtype == FA_DTYPE_F32 ? 4 : dtype == FA_DTYPE_BF16 ? 2 : 1;
  if (((long long)N + 128) * d * es > INT_MAX) return FA_ERR_SHAPE;

  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.descales = descales;
  a.BH = (int)BH;
  a.N = N;
  a.n_qtiles = (int)n_qtiles;
  a.causal = causal ? 1 : 0;
  a.scale = scale;
  const bool c = causal != 0;
  switch (dtype) {
    case FA_DTYPE_BF16:
      return d == 128 ? launch_fwd_dma<fa::kBF16>(a, c, stream)
                      : launch_fwd<fa::kBF16, 64, 64>(a, c, stream);
    case FA_DTYPE_FP8_E4M3:
      return d == 128 ? launch_fwd_dma<fa::kFP8>(a, c, stream)
                      : launch_fwd<fa::kFP8, 64, 64>(a, c, stream);
    default:
      return d == 128 ? launch_fwd<fa::kF32, 128, 32>(a, c, stream)
                      : launch_fwd<fa::kF32, 64, 32>(a, c, stream);
  }
}

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
    if (in_dtype == FA_DTYPE_BF16) {
      hipLaunchKernelGGL(fa::fa_amax_kernel<true>, grid, dim3(256), 0, stream, x, amax, per_head);
      hipLaunchKernelGGL(fa::fa_quant_kernel<true>, grid, dim3(256), 0, stream, x,
                         (uint8_t*)x_fp8, (const uint32_t*)amax, per_head);
    } else {
      hipLaunchKernelGGL(fa::fa_amax_kernel<false>, grid, dim3(256), 0, stream, x, amax, per_head);
      hipLaunchKernelGGL(fa::fa_quant_kernel<false>, grid, dim3(256), 0, stream, x,
                         (uint8_t*)x_fp8, (const uint32_t*)amax, per_head);
    }
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  }
  hipLaunchKernelGGL(fa::fa_descale_finalize, dim3((nbh + 255) / 256), dim3(256), 0, stream, amax,
                     nbh);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
