// C ABI of libfa.so, forward part: argument validation, choice of kernel
// instantiation, and launch on the caller's stream for the forward, split-KV
// and merge entry points (the quantisers are in fa_quant_api.hip, the backward
// in fa_bwd_api.hip). The declarations and the contract of every entry point
// are in include/fa.h.
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa.h"
#include "fa_api_common.hpp"
#include "fa_api_device.hpp"
#include "fa_fwd_kernel.hpp"
#include "fa_merge_kernel.hpp"

namespace {

using fa_api::aligned16;
using fa_api::aligned4;
using fa_api::ceil_div;

// Every kernel: 4 waves x 32 query rows per workgroup. The register-staged
// kernel (fp32, d = 64 and 128) takes key tile 32, registers bounded so two
// workgroups share a CU (2 waves per SIMD).
constexpr int kWaves = 4;
constexpr int kWavesPerSimd = 2;

// bf16 and fp8: global -> LDS by DMA, V^T read with the LDS transpose reads.
// Head dim 128 has two tile configurations:
//   narrow: key tile 32 (bf16, three stages) / 64 (fp8, two stages), three
//           waves per SIMD, three workgroups per CU (48 / 32 KB of LDS);
//   wide:   key tile 64 (bf16) / 128 (fp8), two stages (64 KB), two waves per
//           SIMD, two workgroups per CU.
// Wide runs grids of at most two workgroups per CU, where a third slot per CU
// would stay empty: the wider tile halves the per-tile barrier, max, rescale
// test and DMA work. Measured against the narrow tiles (same box, medians, L2
// flushed, timing order alternated): unsplit 8 x 4096 bf16 +17%, FP8 +14%,
// 16 x 2048 +16%, 4 x 8192 +17%; on full grids the third wave per SIMD is
// worth more (56 x 30272 bf16 -4.7%, a 768-workgroup grid -2%).
// MX: per-block FP8 scales (fp8 only), narrow tiles.
// Head dim 64 has one configuration, two stages of 32 KB: key tile 64 at four
// waves per SIMD (bf16, about 120 registers) and 128 at three (fp8, about 152).
// Half the Q and O registers of d = 128 leave room for twice the keys per
// tile, which spreads the per-tile work of this VALU-bound head dim over more
// scores. Measured against key tile 32 and against three stages at three
// waves per SIMD (same box, medians, L2 flushed): bf16 56 x 30272 999 against
// 959 / 975 TFLOP/s, 8 x 4096 +4% / +38%.
template <int DT, int D, bool CAUSAL, bool SPLIT, bool MX, bool WIDE>
void launch_fwd_dma_inst(const fa::FwdArgs& a, hipStream_t stream) {
  constexpr bool kB = DT == fa::kBF16;
  constexpr int BN = D == 64 ? (kB ? 64 : 128) : kB ? (WIDE ? 64 : 32) : (WIDE ? 128 : 64);
  constexpr int NSTAGE = D == 128 && kB && !WIDE ? 3 : 2;
  constexpr int LOOK = 2, WPE = D == 64 ? (kB ? 4 : 3) : WIDE ? 2 : 3;
  static_assert(!(MX && WIDE), "per-block FP8 runs the narrow tiles");
  static_assert(D == 128 || !WIDE, "head dim 64: one configuration");
  // FP8: the reference max may lag the running max by 0.75 (log2 units)
  constexpr int TAUQ = DT == fa::kFP8 ? 3 : 0;
  // the prefetch goes out before the QK MFMAs (issuing it after them was
  // measured no faster on any shape, and 2-4% slower for FP8 non-causal)
  constexpr bool LATE = false;
  const long long items = (long long)a.BH * a.n_qtiles * (SPLIT ? a.n_splits : 1);
  hipLaunchKernelGGL((fa::fa_fwd_dma_kernel<DT, BN, kWaves, CAUSAL, LOOK, WPE, NSTAGE, SPLIT, MX, TAUQ, LATE, D>),
                     dim3((unsigned)items), dim3(64 * kWaves), 0, stream, a);
}

template <int DT, int D, bool MX, bool WIDE>
void launch_fwd_dma_cfg(const fa::FwdArgs& a, bool causal, bool split, hipStream_t stream) {
  if (causal)
    split ? launch_fwd_dma_inst<DT, D, true, true, MX, WIDE>(a, stream)
          : launch_fwd_dma_inst<DT, D, true, false, MX, WIDE>(a, stream);
  else
    split ? launch_fwd_dma_inst<DT, D, false, true, MX, WIDE>(a, stream)
          : launch_fwd_dma_inst<DT, D, false, false, MX, WIDE>(a, stream);
}

template <int DT, bool MX = false, int D = 128>
int launch_fwd_dma(const fa::FwdArgs& a, bool causal, bool split, hipStream_t stream) {
  const long long items = (long long)a.BH * a.n_qtiles * (split ? a.n_splits : 1);
  const int cus = fa_api::device_cus();
  if constexpr (MX || D == 64) {
    launch_fwd_dma_cfg<DT, D, MX, false>(a, causal, split, stream);
  } else {
    if (cus > 0 && items <= 2LL * cus)
      launch_fwd_dma_cfg<DT, D, false, true>(a, causal, split, stream);
    else
      launch_fwd_dma_cfg<DT, D, false, false>(a, causal, split, stream);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <int DT, int D, int BN, bool CAUSAL, bool SPLIT>
void launch_fwd_inst(const fa::FwdArgs& a, hipStream_t stream) {
  using C = fa::Cfg<DT, D, BN, kWaves>;
  const long long items = (long long)a.BH * a.n_qtiles * (SPLIT ? a.n_splits : 1);
  hipLaunchKernelGGL((fa::fa_fwd_kernel<DT, D, BN, kWaves, CAUSAL, kWavesPerSimd, 0, SPLIT>),
                     dim3((unsigned)items), dim3(C::NT), 0, stream, a);
}

template <int DT, int D, int BN>
int launch_fwd(const fa::FwdArgs& a, bool causal, bool split, hipStream_t stream) {
  if (causal)
    split ? launch_fwd_inst<DT, D, BN, true, true>(a, stream) : launch_fwd_inst<DT, D, BN, true, false>(a, stream);
  else
    split ? launch_fwd_inst<DT, D, BN, false, true>(a, stream) : launch_fwd_inst<DT, D, BN, false, false>(a, stream);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Kernel choice by dtype and head dim (validated by the caller); mx selects
// the per-block FP8 kernel (fp8, head dim 128).
int launch_any(const fa::FwdArgs& a, int dtype, int d, bool split, bool mx, hipStream_t stream) {
  const bool c = a.causal != 0;
  if (mx) return launch_fwd_dma<fa::kFP8, true>(a, c, split, stream);
  switch (dtype) {
    case FA_DTYPE_BF16:
      return d == 128 ? launch_fwd_dma<fa::kBF16>(a, c, split, stream)
                      : launch_fwd_dma<fa::kBF16, false, 64>(a, c, split, stream);
    case FA_DTYPE_FP8_E4M3:
      return d == 128 ? launch_fwd_dma<fa::kFP8>(a, c, split, stream)
                      : launch_fwd_dma<fa::kFP8, false, 64>(a, c, split, stream);
    default:
      return d == 128 ? launch_fwd<fa::kF32, 128, 32>(a, c, split, stream)
                      : launch_fwd<fa::kF32, 64, 32>(a, c, split, stream);
  }
}

constexpr int kBM = 32 * kWaves;   // query rows per workgroup

// Argument checks shared by fa_fwd and fa_fwd_splitkv, in the documented
// order; fills the kernel arguments. Returns FA_OK with *empty = true when
// there is nothing to compute.
// E8M0 block scales of the per-block FP8 forward (null for the other paths).
struct MxScales {
  const unsigned char* q;
  const unsigned char* k;
  const unsigned char* v;
};

int prepare_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int Hkv, int N, int d, int causal, float scale, int dtype, const float* descales,
                const MxScales* mx, fa::FwdArgs& a, bool& empty);


int prepare_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int Hkv, int N, int d, int causal, float scale, int dtype, const float* descales,
                const MxScales* mx, fa::FwdArgs& a, bool& empty) {
  empty = false;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (H > 0 && (Hkv < 1 || H % Hkv != 0)) return FA_ERR_SHAPE;
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP8_E4M3)
    return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (mx && d != 128) return FA_ERR_HEAD_DIM;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (mx && (!mx->q || !mx->k || !mx->v)) return FA_ERR_DESCALES;
  if (!mx && dtype == FA_DTYPE_FP8_E4M3 && descales == nullptr) return FA_ERR_DESCALES;
  const long long BH = (long long)B * H;
  if (BH == 0 || N == 0) {
    empty = true;
    return FA_OK;
  }
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_ALIGN;
  if (mx && (!aligned4(mx->q) || !aligned4(mx->k) || !aligned4(mx->v))) return FA_ERR_ALIGN;
  const long long n_qtiles = ((long long)N + kBM - 1) / kBM;
  if (BH > INT_MAX || BH * n_qtiles > INT_MAX) return FA_ERR_SHAPE;
  // one head of Q, K or V is addressed with 32-bit buffer offsets
  const long long es = dtype == FA_DTYPE_F32 ? 4 : dtype == FA_DTYPE_BF16 ? 2 : 1;
  if (((long long)N + 128) * d * es > INT_MAX) return FA_ERR_SHAPE;

  a = fa::FwdArgs{};
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
  a.group = H / Hkv;
  a.causal_order = fa_api::causal_order(BH, a.group, N, d, es);
  if (mx) {
    a.q_scale = mx->q;
    a.k_scale = mx->k;
    a.v_scale = mx->v;
  }
  return FA_OK;
}

// Compute units of the current device, cached per device (0 if the query fails).
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
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: split-KV workspace missing, misaligned or too small";
    case FA_ERR_SPLITS: return "FA_ERR_SPLITS: number of splits / parts must be 1..FA_MAX_SPLITS";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the partials need more than the library's static scratch (FA_STATIC_SCRATCH_BYTES)";
    default: return "unknown fa status";
  }
}

namespace {

// The forward behind every entry point: Hq query heads over Hkv key/value
// heads; num_splits == 0 runs the unsplit kernels (no workspace), >= 1 the
// split-KV kernels and the merge in `workspace`.
int run_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
            int Hkv, int N, int d, int causal, float scale, int dtype, const float* descales,
            const MxScales* mx, int num_splits, void* workspace, size_t workspace_bytes,
            hipStream_t stream) {
  fa::FwdArgs a;
  bool empty = false;
  const int st = prepare_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, descales, mx, a, empty);
  if (st != FA_OK) return st;
  if (num_splits == 0) return empty ? FA_OK : launch_any(a, dtype, d, false, mx != nullptr, stream);
  if (num_splits < 1 || num_splits > FA_MAX_SPLITS) return FA_ERR_SPLITS;
  if (empty) return FA_OK;
  const size_t need = fa_splitkv_workspace_bytes(B, Hq, N, d, num_splits);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return FA_ERR_WORKSPACE;
  const int chunk = fa_splitkv_chunk_keys(N, num_splits);
  const int used = (int)ceil_div(N, chunk);               // chunks that hold keys
  if ((long long)a.BH * a.n_qtiles * used > INT_MAX) return FA_ERR_SHAPE;
  float* o_parts = static_cast<float*>(workspace);
  float* lse_parts = o_parts + (size_t)num_splits * a.BH * (size_t)N * d;
  a.n_splits = used;
  a.split_keys = chunk;
  a.o_part = o_parts;
  a.lse_part = lse_parts;
  const int r = launch_any(a, dtype, d, true, mx != nullptr, stream);
  if (r != FA_OK) return r;
  return fa_merge_partials(o_parts, lse_parts, used, B, Hq, N, d,
                           dtype == FA_DTYPE_F32 ? FA_DTYPE_F32 : FA_DTYPE_BF16, o, lse, stream);
}

}  // namespace

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int d, int causal, float scale, int dtype,
                      const float* descales, hipStream_t stream) {
  return run_fwd(q, k, v, o, lse, B, H, H, N, d, causal, scale, dtype, descales, nullptr, 0, nullptr, 0,
                 stream);
}

extern "C" int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int N, int d, int causal, float scale, int dtype,
                          const float* descales, int num_splits, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  if (num_splits < 1 || num_splits > FA_MAX_SPLITS) {
    // shape and argument errors come first, as for the other entry points
    fa::FwdArgs a;
    bool empty = false;
    const int st = prepare_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, descales, nullptr,
                               a, empty);
    return st != FA_OK ? st : FA_ERR_SPLITS;
  }
  return run_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, descales, nullptr,
                 num_splits == 1 ? 0 : num_splits, workspace, workspace_bytes, stream);
}

extern "C" int fa_fwd_mxfp8(const void* q, const void* k, const void* v, const unsigned char* q_scales,
                            const unsigned char* k_scales, const unsigned char* v_scales, void* o,
                            float* lse, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                            int num_splits, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const MxScales mx{q_scales, k_scales, v_scales};
  if (num_splits < 1 || num_splits > FA_MAX_SPLITS) {
    fa::FwdArgs a;
    bool empty = false;
    const int st = prepare_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, FA_DTYPE_FP8_E4M3, nullptr,
                               &mx, a, empty);
    return st != FA_OK ? st : FA_ERR_SPLITS;
  }
  return run_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, FA_DTYPE_FP8_E4M3, nullptr, &mx,
                 num_splits == 1 ? 0 : num_splits, workspace, workspace_bytes, stream);
}

extern "C" int fa_splitkv_chunk_keys(int N, int num_splits) {
  if (N <= 0 || num_splits < 1 || num_splits > FA_MAX_SPLITS) return 0;
  const long long per = ceil_div(N, num_splits);
  return (int)(ceil_div(per, 128) * 128);
}

extern "C" size_t fa_splitkv_workspace_bytes(int B, int H, int N, int d, int num_splits) {
  if (B < 0 || H < 0 || N < 0 || (d != 64 && d != 128)) return 0;
  if (num_splits < 1 || num_splits > FA_MAX_SPLITS) return 0;
  return (size_t)4 * (size_t)num_splits * (size_t)B * (size_t)H * (size_t)N * (size_t)(d + 1);
}

extern "C" int fa_splitkv_default_splits(int B, int H, int N, int d, int causal, int dtype) {
  if (B <= 0 || H <= 0 || N <= 0) return 1;
  if (d != 64 && d != 128) return 1;
  const int cus = fa_api::device_cus();
  if (cus <= 0) return 1;
  return fa_api::default_splits((long long)B * H * ceil_div(N, kBM), N, causal != 0, cus,
                                dtype == FA_DTYPE_FP8_E4M3);
}

extern "C" int fa_merge_partials(const float* o_parts, const float* lse_parts, int num_parts,
                                 int B, int H, int N, int d, int out_dtype, void* o, float* lse,
                                 hipStream_t stream) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (out_dtype != FA_DTYPE_F32 && out_dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (num_parts < 1 || num_parts > FA_MAX_SPLITS) return FA_ERR_SPLITS;
  const long long rows = (long long)B * H * N;
  if (rows == 0) return FA_OK;
  if (!o_parts || !lse_parts || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(o_parts) || !aligned16(o)) return FA_ERR_ALIGN;
  const int rpb = 256 / (d / 4);
  const long long blocks = ceil_div(rows, rpb);
  if (blocks > INT_MAX) return FA_ERR_SHAPE;
  const dim3 grid((unsigned)blocks), block(256);
  if (d == 128) {
    if (out_dtype == FA_DTYPE_F32)
      hipLaunchKernelGGL((fa::fa_merge_kernel<128, true>), grid, block, 0, stream, o_parts, lse_parts,
                         num_parts, rows, o, lse);
    else
      hipLaunchKernelGGL((fa::fa_merge_kernel<128, false>), grid, block, 0, stream, o_parts, lse_parts,
                         num_parts, rows, o, lse);
  } else {
    if (out_dtype == FA_DTYPE_F32)
      hipLaunchKernelGGL((fa::fa_merge_kernel<64, true>), grid, block, 0, stream, o_parts, lse_parts,
                         num_parts, rows, o, lse);
    else
      hipLaunchKernelGGL((fa::fa_merge_kernel<64, false>), grid, block, 0, stream, o_parts, lse_parts,
                         num_parts, rows, o, lse);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int N, int d, int causal, float scale, int dtype,
                              const float* descales, int num_splits, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  if (num_splits == 0) num_splits = -1;   // 0 selects the unsplit path inside run_fwd
  return run_fwd(q, k, v, o, lse, B, H, H, N, d, causal, scale, dtype, descales, nullptr, num_splits,
                 workspace, workspace_bytes, stream);
}

// Scratch of fa_fwd_splitkv_static: the split-KV partials of one call, in the
// library's own device memory, so that the call allocates nothing. Every
// device the library runs on holds its own copy from the first use of the
// library there until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: host code only ever passes the
// per-device address taken below.
static __device__ __align__(256) unsigned char scratch[FA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_HIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FA_OK;
}

}  // namespace

extern "C" int fa_fwd_splitkv_static(const void* q, const void* k, const void* v, void* o, float* lse,
                                     int B, int H, int N, int d, int causal, float scale, int dtype,
                                     const float* descales, int num_splits, hipStream_t stream) {
  // the argument errors of fa_fwd_splitkv, in its order, before the scratch check
  fa::FwdArgs a;
  bool empty = false;
  const int st = prepare_fwd(q, k, v, o, lse, B, H, H, N, d, causal, scale, dtype, descales, nullptr, a, empty);
  if (st != FA_OK) return st;
  if (num_splits < 1 || num_splits > FA_MAX_SPLITS) return FA_ERR_SPLITS;
  if (empty) return FA_OK;
  const size_t need = fa_splitkv_workspace_bytes(B, H, N, d, num_splits);
  if (need > (size_t)FA_STATIC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  const int r = scratch_address(&ws);
  if (r != FA_OK) return r;
  return run_fwd(q, k, v, o, lse, B, H, H, N, d, causal, scale, dtype, descales, nullptr, num_splits, ws,
                 (size_t)FA_STATIC_SCRATCH_BYTES, stream);
}
