// Test helper (not part of libfa): the head-dim-128 forward kernel the library
// launches, in its narrow (key tile 32 bf16 / 64 FP8, three waves per SIMD) or
// wide (64 / 128, two waves per SIMD) tile configuration, instantiated with
// other LDS pipeline depths (NSTAGE), other MFMA operand look-ahead (LOOK) and
// the prefetch issued before or after the QK MFMAs (LATE). None of them changes any arithmetic or its order, only when
// tiles land in LDS and when operands are read, so every variant must give
// the library's outputs bit for bit: the race detector of the determinism
// tests (a missing wait or barrier shows up as a difference).
#include <hip/hip_runtime.h>

#include "fa.h"
#include "fa_api_common.hpp"
#include "fa_fwd_kernel.hpp"

namespace {

template <int DT, bool CAUSAL, int NSTAGE, int LOOK, bool LATE, bool WIDE>
void launch(const fa::FwdArgs& a, hipStream_t stream) {
  constexpr int BN = DT == fa::kBF16 ? (WIDE ? 64 : 32) : (WIDE ? 128 : 64);
  constexpr int WPE = WIDE ? 2 : 3;
  constexpr int TAUQ = DT == fa::kFP8 ? 3 : 0;
  hipLaunchKernelGGL((fa::fa_fwd_dma_kernel<DT, BN, 4, CAUSAL, LOOK, WPE, NSTAGE, false, false, TAUQ, LATE>),
                     dim3((unsigned)(a.BH * a.n_qtiles)), dim3(256), 0, stream, a);
}

template <int DT, bool CAUSAL, bool LATE, bool WIDE>
int pick_late(const fa::FwdArgs& a, int nstage, int look, hipStream_t stream) {
  if (nstage == 2 && look == 1) launch<DT, CAUSAL, 2, 1, LATE, WIDE>(a, stream);
  else if (nstage == 2 && look == 2) launch<DT, CAUSAL, 2, 2, LATE, WIDE>(a, stream);
  else if (nstage == 3 && look == 1) launch<DT, CAUSAL, 3, 1, LATE, WIDE>(a, stream);
  else if (nstage == 3 && look == 2) launch<DT, CAUSAL, 3, 2, LATE, WIDE>(a, stream);
  else return FA_ERR_SHAPE;
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <int DT, bool CAUSAL>
int pick(const fa::FwdArgs& a, int nstage, int look, int late, int wide, hipStream_t stream) {
  if (wide)
    return late ? pick_late<DT, CAUSAL, true, true>(a, nstage, look, stream)
                : pick_late<DT, CAUSAL, false, true>(a, nstage, look, stream);
  return late ? pick_late<DT, CAUSAL, true, false>(a, nstage, look, stream)
              : pick_late<DT, CAUSAL, false, false>(a, nstage, look, stream);
}

}  // namespace

// The forward of fa_fwd (d = 128, bf16 or FP8, unsplit) in the narrow (wide =
// 0) or wide (1) tile configuration with the given LDS stage count (2 or 3),
// operand look-ahead (1 or 2) and prefetch order (late = after the QK MFMAs).
// Same arguments and layouts as fa_fwd; N >= 1, B*H >= 1, 16-byte aligned
// tensors (the tests pass torch allocations).
extern "C" int fa_test_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                   int H, int N, int causal, float scale, int dtype, const float* descales,
                                   int nstage, int look, int late, int wide, hipStream_t stream) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP8_E4M3) return FA_ERR_DTYPE;
  if (!q || !k || !v || !o || !lse || (dtype == FA_DTYPE_FP8_E4M3 && !descales)) return FA_ERR_NULL;
  const long long es = dtype == FA_DTYPE_BF16 ? 2 : 1;
  if (((long long)N + 128) * 128 * es > 0x7fffffffLL) return FA_ERR_SHAPE;
  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.descales = descales;
  a.BH = B * H;
  a.N = N;
  a.n_qtiles = (N + 127) / 128;
  a.causal = causal ? 1 : 0;
  a.scale = scale;
  a.group = 1;
  a.causal_order = fa_api::causal_order(a.BH, 1, N, 128, es);
  if (dtype == FA_DTYPE_BF16)
    return causal ? pick<fa::kBF16, true>(a, nstage, look, late, wide, stream)
                  : pick<fa::kBF16, false>(a, nstage, look, late, wide, stream);
  return causal ? pick<fa::kFP8, true>(a, nstage, look, late, wide, stream)
                : pick<fa::kFP8, false>(a, nstage, look, late, wide, stream);
}
