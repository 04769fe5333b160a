/*
 * fa.h -- C ABI of the MI355X (gfx950) FlashAttention-2 forward library,
 * libfa.so.
 *
 * The library computes, for every (batch, head), O = softmax(scale * Q K^T) V
 * and the per-row logsumexp L of the scaled scores. It does this tile by tile
 * with an online softmax (running max m, running sum l, rescale of O by
 * exp(m_old - m_new), one divide by l at the end), so the N x N score matrix
 * never reaches device memory.
 *   - "FlashAttention-2 from PyTorch to Triton", the forward-pass section and
 *     the Triton kernel walkthrough: the algorithm, the L output, the query-tile
 *     grid, and masking of keys past the end.
 *   - "1.8x Faster Attention on an RTX 5080", sections "Who am I, what's
 *     mine?" through "After the last strip: divide, write": the FP8 variant
 *     with per-head descales folded into qk_scale and pv_scale, and P scaled
 *     by 256 before it is rounded to FP8.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers on the current HIP device. The
 *     caller allocates and owns them. The library allocates nothing, keeps no
 *     per-call state and never synchronises the host.
 *   - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *     once it is enqueued. Device faults surface at the caller's next
 *     synchronisation.
 *   - Arguments are validated before anything is launched. A negative
 *     fa_status_t is returned on error and nothing is enqueued.
 *   - Offsets are computed in 64 bits; B*H*N*d may exceed 2^31.
 */
#ifndef FA_H_
#define FA_H_

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_DTYPE_F32 = 0,      /* fp32 inputs, fp32 O, fp32 MFMA products (no reduced precision) */
  FA_DTYPE_BF16 = 1,     /* bf16 inputs, bf16 O, fp32 accumulation                         */
  FA_DTYPE_FP8_E4M3 = 2  /* OCP e4m3fn inputs + fp32 descales, bf16 O, fp32 accumulation   */
} fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,      /* a required pointer is NULL                          */
  FA_ERR_SHAPE = -2,     /* B, H or N negative                                  */
  FA_ERR_DTYPE = -3,     /* unknown dtype code                                  */
  FA_ERR_HEAD_DIM = -4,  /* d is not 64 or 128                                  */
  FA_ERR_SCALE = -5,     /* scale is NaN or infinite                            */
  FA_ERR_DESCALES = -6,  /* FP8 requested without a descale array               */
  FA_ERR_ALIGN = -7,     /* a tensor pointer is not 16-byte aligned             */
  FA_ERR_HIP = -8        /* the HIP runtime rejected a launch                   */
} fa_status_t;

/*
 * fa_fwd -- the FlashAttention-2 forward pass.
 *
 *   q, k, v  [B, H, N, d] contiguous, element type by `dtype`:
 *            FA_DTYPE_F32 -> float, FA_DTYPE_BF16 -> bfloat16,
 *            FA_DTYPE_FP8_E4M3 -> one byte per element (e4m3fn code).
 *   o        [B, H, N, d] contiguous output; float for FA_DTYPE_F32,
 *            bfloat16 otherwise.
 *   lse      [B, H, N] contiguous float output: the natural-log logsumexp of
 *            the scaled scores of each query row (for FP8: of the dequantised
 *            scores), L_i = log sum_j exp(S_ij).
 *   B, H, N  batch, heads, sequence length (queries = keys = N). N == 0 or
 *            B*H == 0 returns FA_OK without launching.
 *   d        head dimension, 64 or 128.
 *   causal   non-zero: key j is seen by query i only if j <= i.
 *   scale    multiplies Q K^T; any finite value (callers pass 1/sqrt(d)).
 *   dtype    a fa_dtype_t.
 *   descales FA_DTYPE_FP8_E4M3 only (ignored otherwise): device float
 *            [3][B*H], rows q, k, v. The kernel uses
 *            qk_scale = scale * dq * dk and multiplies the output by
 *            dv / 256 / l, undoing the x256 applied to P before its FP8
 *            rounding.
 *   stream   HIP stream to enqueue on.
 *
 * Keys at index >= N are excluded, not zero-padded; query rows >= N of the
 * last tile are computed on zeros and never stored.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, int causal, float scale, int dtype,
           const float* descales, hipStream_t stream);

/*
 * fa_quantize_fp8 -- per-head FP8 quantisation of one tensor
 * ("1.8x Faster Attention on an RTX 5080", section "Who am I, what's mine?":
 * FP8 Q, K and V with one fp32 descale per head).
 *
 *   x        [B, H, N, d] contiguous, float (in_dtype FA_DTYPE_F32) or
 *            bfloat16 (FA_DTYPE_BF16).
 *   x_fp8    [B, H, N, d] contiguous output, one e4m3fn code per element.
 *   descale  [B*H] device float output: amax / 448 per (batch, head)
 *            (1 for an all-zero head).
 *   Per (batch, head): amax = max |x| in fp32; mult = 448 / amax (correctly
 *   rounded fp32 division); code = e4m3 round-to-nearest-even of
 *   clamp(x * mult, -448, 448).
 *   The descale array is also the amax accumulator while the call runs: the
 *   three kernels it enqueues must not overlap another use of that array.
 */
int fa_quantize_fp8(const void* x, int in_dtype, void* x_fp8, float* descale,
                    int B, int H, int N, int d, hipStream_t stream);

/* Human-readable name of a fa_status_t value. Never NULL. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
