// Test helper (not part of libfa): the forward DMA kernel the library launches
// at head dim 128, in its narrow (key tile 32 bf16 / 64 FP8, three waves per
// SIMD) or wide (64 / 128, two waves per SIMD) tile configuration, or at head
// dim 64 (64 / 128, four / three waves per SIMD), instantiated with
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

// CFG 0: d = 128 narrow, 1: d = 128 wide, 2: d = 64
template <int DT, bool CAUSAL, int NSTAGE, int LOOK, bool LATE, int CFG>
void launch(const fa::FwdArgs& a, hipStream_t stream) {
  constexpr int D = CFG == 2 ? 64 : 128;
  constexpr int BN = DT == fa::kBF16 ? (CFG == 0 ? 32 : 64) : (CFG == 0 ? 64 : 128);
  constexpr int WPE = CFG == 1 ? 2 : CFG == 2 && DT == fa::kBF16 ? 4 : 3;
  constexpr int TAUQ = DT == fa::kFP8 ? 3 : 0;
  hipLaunchKernelGGL((fa::fa_fwd_dma_kernel<DT, BN, 4, CAUSAL, LOOK, WPE, NSTAGE, false, false, TAUQ, LATE, D>),
                     dim3((unsigned)(a.BH * a.n_qtiles)), dim3(256), 0, stream, a);
}

template <int DT, bool CAUSAL, bool LATE, int CFG>
int pick_late(const fa::FwdArgs& a, int nstage, int look, hipStream_t stream) {
  if (nstage == 2 && look == 1) launch<DT, CAUSAL, 2, 1, LATE, CFG>(a, stream);
  else if (nstage == 2 && look == 2) launch<DT, CAUSAL, 2, 2, LATE, CFG>(a, stream);
  else if (nstage == 3 && look == 1) launch<DT, CAUSAL, 3, 1, LATE, CFG>(a, stream);
  else if (nstage == 3 && look == 2) launch<DT, CAUSAL, 3, 2, LATE, CFG>(a, stream);
  else return FA_ERR_SHAPE;
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <int DT, bool CAUSAL, int CFG>
int pick_cfg(const fa::FwdArgs& a, int nstage, int look, int late, hipStream_t stream) {
  return late ? pick_late<DT, CAUSAL, true, CFG>(a, nstage, look, stream)
              : pick_late<DT, CAUSAL, false, CFG>(a, nstage, look, stream);
}

template <int DT, bool CAUSAL>
int pick(const fa::FwdArgs& a, int d, int nstage, int look, int late, int wide, hipStream_t stream) {
  if (d == 64) return pick_cfg<DT, CAUSAL, 2>(a, nstage, look, late, stream);
  return wide ? pick_cfg<DT, CAUSAL, 1>(a, nstage, look, late, stream)
              : pick_cfg<DT, CAUSAL, 0>(a, nstage, look, late, stream);
}

}  // namespace

// The forward of fa_fwd (bf16 or FP8, unsplit) at head dim d = 128, in the
// narrow (wide = 0) or wide (1) tile configuration, or at d = 64 (wide
// ignored), with the given LDS stage count (2 or 3), operand look-ahead (1 or
// 2) and prefetch order (late = after the QK MFMAs). Same arguments and
// layouts as fa_fwd; N >= 1, B*H >= 1, 16-byte aligned tensors (the tests pass
// torch allocations).
extern "C" int fa_test_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                   int H, int N, int d, int causal, float scale, int dtype,
                                   const float* descales, int nstage, int look, int late, int wide,
                                   hipStream_t stream) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP8_E4M3) return FA_ERR_DTYPE;
  if (!q || !k || !v || !o || !lse || (dtype == FA_DTYPE_FP8_E4M3 && !descales)) return FA_ERR_NULL;
  const long long es = dtype == FA_DTYPE_BF16 ? 2 : 1;
  if (((long long)N + 128) * d * es > 0x7fffffffLL) return FA_ERR_SHAPE;
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
  a.causal_order = fa_api::causal_order(a.BH, 1, N, d, es);
  if (dtype == FA_DTYPE_BF16)
    return causal ? pick<fa::kBF16, true>(a, d, nstage, look, late, wide, stream)
                  : pick<fa::kBF16, false>(a, d, nstage, look, late, wide, stream);
  return causal ? pick<fa::kFP8, true>(a, d, nstage, look, late, wide, stream)
                : pick<fa::kFP8, false>(a, d, nstage, look, late, wide, stream);
}
