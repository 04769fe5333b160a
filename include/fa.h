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
 *     per-call state and never synchronises the host (fa_fwd_splitkv_static
 *     alone uses memory of the library's own: a fixed device array).
 *   - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *     once it is enqueued. Device faults surface at the caller's next
 *     synchronisation.
 *   - Arguments are validated before anything is launched. A negative
 *     fa_status_t is returned on error and nothing is enqueued.
 *   - Offsets are computed in 64 bits; B*H*N*d may exceed 2^31.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

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
  FA_ERR_SHAPE = -2,     /* B, H or N negative, heads not a multiple of KV heads, or too large */
  FA_ERR_DTYPE = -3,     /* unknown dtype code                                  */
  FA_ERR_HEAD_DIM = -4,  /* d is not 64 or 128                                  */
  FA_ERR_SCALE = -5,     /* scale is NaN or infinite                            */
  FA_ERR_DESCALES = -6,  /* FP8 requested without a descale array               */
  FA_ERR_ALIGN = -7,     /* a tensor pointer is not 16-byte aligned             */
  FA_ERR_HIP = -8,       /* the HIP runtime rejected a launch                   */
  FA_ERR_WORKSPACE = -9, /* split-KV workspace NULL, misaligned or too small    */
  FA_ERR_SPLITS = -10,   /* num_splits / num_parts outside 1..FA_MAX_SPLITS     */
  FA_ERR_SCRATCH = -11   /* fa_fwd_splitkv_static: partials above FA_STATIC_SCRATCH_BYTES */
} fa_status_t;

/* Largest number of key chunks fa_fwd_splitkv and fa_merge_partials accept. */
#define FA_MAX_SPLITS 64

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
 *            B*H == 0 returns FA_OK without launching. One head is
 *            addressed with 32-bit byte offsets: (N + 128) * d * (bytes per
 *            element) above INT_MAX returns FA_ERR_SHAPE (bf16, d = 128:
 *            N <= 8388479), as does B*H*ceil(N/128) above INT_MAX.
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

/*
 * fa_quantize_fp8_rotated -- randomised Hadamard rotation, then per-head FP8
 * quantisation ("Kernels and Memory in LLM Inference", section "Precision:
 * FP8 with a real failure mode": a fixed random rotation of Q and K before
 * quantising spreads the few large outlier coordinates over all dimensions,
 * and the rotations cancel in Q K^T).
 *
 *   x        [B, H, N, d] contiguous bfloat16 (in_dtype FA_DTYPE_BF16 only;
 *            anything else returns FA_ERR_DTYPE), d = 64 or 128.
 *   signs    [d] device int8: a negative entry flips that coordinate, any
 *            other value keeps it. Q and K must be rotated with the same signs.
 *   x_fp8    [B, H, N, d] contiguous output codes (e4m3fn) of y = (x * s) H,
 *            H the unnormalised d x d Sylvester Hadamard matrix
 *            (H_ij = (-1)^popcount(i & j), H H^T = d I). y is computed in
 *            float64 (exact for bf16 rows spanning at most 38 binary orders
 *            of magnitude) and rounded once to fp32, then quantised per head
 *            exactly as fa_quantize_fp8 does.
 *   descale  [B*H] device float output: amax(y) / 448 per (batch, head), 1 for
 *            an all-zero head, times 1/d when fold_inverse_d is non-zero.
 *            Rotate Q with fold_inverse_d = 1 and K with 0: the FP8 forward
 *            then computes the same attention, since (Q s H)(K s H)^T = d Q K^T.
 *   Both pointers of x and x_fp8 must be 16-byte aligned (FA_ERR_ALIGN). The
 *   descale array is the amax accumulator while the call runs, as for
 *   fa_quantize_fp8. Errors are returned before anything is enqueued.
 */
int fa_quantize_fp8_rotated(const void* x, int in_dtype, const signed char* signs, void* x_fp8,
                            float* descale, int B, int H, int N, int d, int fold_inverse_d,
                            hipStream_t stream);

/*
 * Per-block FP8 ("Kernels and Memory in LLM Inference", section "Precision:
 * FP8 with a real failure mode": one scale per block of values, so that an
 * outlier widens only its own block's grid instead of the whole tensor's).
 *
 * A block is 32 consecutive elements along the axis the product it feeds
 * sums over, as in the OCP microscaling (MX) formats: 32 elements of one row
 * for Q and K (S = Q K^T sums over d), 32 keys of one column for V (O = P V
 * sums over the keys; the last block of a head holds the N mod 32 keys that
 * remain). Each block has a power-of-two scale 2^e stored as the E8M0 byte
 * e + 127, where e is the smallest integer with amax(block) <= 448 * 2^e
 * (nothing saturates), clamped to [-127, 127] (an all-zero block gets 0x00);
 * the codes are e4m3fn round-to-nearest-even of x * 2^-e, and the value of a
 * code is its e4m3 value times 2^e. Non-finite inputs give unspecified codes.
 */

/*
 * fa_quantize_mxfp8_rows -- row blocks (for Q and K).
 *   x        [B, H, N, d] contiguous float (FA_DTYPE_F32) or bfloat16
 *            (FA_DTYPE_BF16), d = 64 or 128, 16-byte aligned.
 *   signs    NULL, or [d] device int8: the input rows are first rotated by
 *            the randomised Hadamard transform of fa_quantize_fp8_rotated
 *            (exact float64 sums rounded once to fp32; bfloat16 input only,
 *            else FA_ERR_DTYPE).
 *   fold_inverse_d  non-zero: the (rotated) values are multiplied by the
 *            power of two 1/d in fp32 before quantising (for a rotated Q).
 *   x_fp8    [B, H, N, d] contiguous e4m3fn codes, 16-byte aligned.
 *   scales   [B, H, N, d/32] E8M0 bytes.
 * One pass; every block is independent. Returns before launching on errors.
 */
int fa_quantize_mxfp8_rows(const void* x, int in_dtype, const signed char* signs, int fold_inverse_d,
                           void* x_fp8, unsigned char* scales, int B, int H, int N, int d,
                           hipStream_t stream);

/*
 * fa_quantize_mxfp8_keys -- key blocks (for V).
 *   x        [B, H, N, d] contiguous float or bfloat16, 16-byte aligned.
 *   x_fp8    [B, H, N, d] contiguous e4m3fn codes, 16-byte aligned.
 *   scales   [B, H, ceil(N/32), d] E8M0 bytes, 4-byte aligned: the scale of
 *            keys 32c .. 32c + 31 of column j at [b][h][c][j].
 */
int fa_quantize_mxfp8_keys(const void* x, int in_dtype, void* x_fp8, unsigned char* scales,
                           int B, int H, int N, int d, hipStream_t stream);

/*
 * fa_fwd_mxfp8 -- the FP8 forward on per-block codes. The block scales are
 * applied inside gfx950's scaled matrix instructions (no extra arithmetic per
 * score); the softmax, P's FP8 rounding and the outputs are those of fa_fwd
 * with dtype FA_DTYPE_FP8_E4M3, with the dequantised values
 * code * 2^(scale - 127) in place of code * descale.
 *   q         [B, Hq, N, d] codes with q_scales [B, Hq, N, d/32];
 *   k         [B, Hkv, N, d] codes with k_scales [B, Hkv, N, d/32];
 *   v         [B, Hkv, N, d] codes with v_scales [B, Hkv, ceil(N/32), d];
 *             Hq a multiple of Hkv (query head h reads K/V head h / (Hq/Hkv)).
 *   o, lse    as fa_fwd (bf16 O [B, Hq, N, d], fp32 L [B, Hq, N]).
 *   d must be 128 (FA_ERR_HEAD_DIM otherwise). Missing scale arrays return
 *   FA_ERR_DESCALES, scale arrays not 4-byte aligned FA_ERR_ALIGN.
 *   num_splits 1 runs unsplit (workspace unused); 2..FA_MAX_SPLITS run the
 *   split-KV path with the workspace of fa_fwd_splitkv.
 */
int fa_fwd_mxfp8(const void* q, const void* k, const void* v, const unsigned char* q_scales,
                 const unsigned char* k_scales, const unsigned char* v_scales, void* o, float* lse,
                 int B, int Hq, int Hkv, int N, int d, int causal, float scale, int num_splits,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Split-KV forward ("Kernels and Memory in LLM Inference", section
 * "Flash-Decoding: one token, whole chip": cut the keys into contiguous
 * chunks, give every chunk its own workgroup with its own running max and sum,
 * and merge the partial results in a second kernel by rescaling each to the
 * overall max). It multiplies the number of workgroups when B*H*ceil(N/128)
 * alone cannot fill the device. The result is the same attention as fa_fwd,
 * up to rounding.
 */

/*
 * fa_splitkv_chunk_keys -- keys per chunk when the keys are cut into
 * num_splits chunks: chunk = 128 * ceil(ceil(N / num_splits) / 128). Chunk s
 * covers the keys [s * chunk, min(N, (s + 1) * chunk)); only the first
 * ceil(N / chunk) <= num_splits chunks hold keys. Returns 0 when N <= 0 or
 * num_splits is outside 1..FA_MAX_SPLITS.
 */
int fa_splitkv_chunk_keys(int N, int num_splits);

/*
 * fa_splitkv_workspace_bytes -- device workspace fa_fwd_splitkv needs:
 * 4 * num_splits * B*H * N * (d + 1) bytes. Returns 0 for invalid arguments
 * (negative sizes, d not 64 or 128, num_splits outside 1..FA_MAX_SPLITS).
 */
size_t fa_splitkv_workspace_bytes(int B, int H, int N, int d, int num_splits);

/*
 * fa_splitkv_default_splits -- the num_splits this library picks for a shape
 * on the current device, with C compute units and W = B*H*ceil(N/128)
 * workgroups of fa_fwd: 1 when W >= 2C; else ceil(2C / W) (non-causal) or
 * ceil(3C / W) (causal), at most N / 1024 (no chunk under 1024 keys; for a
 * non-causal grid with W >= C, N / 2048, or N / 4096 when dtype is
 * FA_DTYPE_FP8_E4M3) and at most 16. Always returns a value >= 1 (1 for
 * invalid arguments or a failed device query).
 */
int fa_splitkv_default_splits(int B, int H, int N, int d, int causal, int dtype);

/*
 * fa_fwd_splitkv -- the forward pass computed chunk by chunk, then merged.
 *
 *   q ... descales  as fa_fwd (same layouts, dtypes and validation).
 *   num_splits      1..FA_MAX_SPLITS; chunks as fa_splitkv_chunk_keys.
 *   workspace       device memory owned by the caller, 16-byte aligned, at
 *                   least fa_splitkv_workspace_bytes(B, H, N, d, num_splits)
 *                   bytes. After the call (stream-ordered) it holds the
 *                   partial results of the written chunks s < ceil(N / chunk):
 *                     o_parts   float [num_splits][B*H][N][d] from byte 0:
 *                               chunk s's output divided by the chunk's own
 *                               softmax sum (already multiplied by the V
 *                               descale for FP8);
 *                     lse_parts float [num_splits][B*H][N] right after
 *                               o_parts: the chunk's natural-log logsumexp of
 *                               the scaled scores, -inf for a row with no valid
 *                               key in the chunk (its o_parts row is then 0).
 *   workspace_bytes size of `workspace`, checked against the need.
 *
 * Enqueues two kernels: the chunked forward, then the merge of
 * fa_merge_partials over the written chunks into o and lse. Calls sharing a
 * workspace must not overlap.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, int causal, float scale, int dtype,
                   const float* descales, int num_splits, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/* Size of the library's own device scratch behind fa_fwd_splitkv_static. */
#define FA_STATIC_SCRATCH_BYTES (64u << 20)

/*
 * fa_fwd_splitkv_static -- fa_fwd_splitkv with its partials in the library's
 * own device memory instead of a caller's workspace. For callers that cannot
 * allocate device memory around the call (code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid hipMalloc): the call
 * itself allocates nothing.
 *
 *   q ... num_splits  as fa_fwd_splitkv (same layouts, dtypes, validation
 *                     and error codes, in the same order), then
 *                     FA_ERR_SCRATCH when
 *                     fa_splitkv_workspace_bytes(B, H, N, d, num_splits)
 *                     exceeds FA_STATIC_SCRATCH_BYTES (64 MiB: e.g. 8 heads
 *                     of 4096 tokens, d = 128, in 3 chunks); nothing is
 *                     enqueued then.
 *
 * The scratch is a fixed array in the library's device code: every device the
 * library runs on holds 64 MiB of it until the process ends, and the first
 * call on a device looks up its address there (FA_ERR_HIP if that fails).
 * Every call on one device shares that device's scratch: calls on the same
 * stream are ordered, calls that overlap on one device (other streams, other
 * threads without ordering) race on it. Nothing in it needs clearing: each
 * call writes every partial the merge reads. O and L as fa_fwd_splitkv
 * computes them, bit for bit.
 */
int fa_fwd_splitkv_static(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int N, int d, int causal, float scale, int dtype,
                          const float* descales, int num_splits, hipStream_t stream);

/*
 * fa_merge_partials -- merge attention results computed over disjoint sets of
 * keys (the second kernel of the same section). Per (batch*head, row):
 *   M = max_s L_s,  w_s = exp(L_s - M),  O = sum_s w_s O_s / sum_s w_s,
 *   L = M + log sum_s w_s;
 * parts with L_s = -inf weigh nothing, and a row whose parts are all -inf gets
 * O = 0 and L = -inf.
 *
 *   o_parts    float [num_parts][B*H][N][d], 16-byte aligned: each part's
 *              output divided by its own softmax sum.
 *   lse_parts  float [num_parts][B*H][N]: each part's natural-log logsumexp.
 *   num_parts  1..FA_MAX_SPLITS.
 *   d          64 or 128.
 *   out_dtype  FA_DTYPE_F32 (float O) or FA_DTYPE_BF16 (bfloat16 O).
 *   o          [B*H][N][d] output, 16-byte aligned; lse [B*H][N] output.
 *
 * Parts may come from anywhere (fa_fwd_splitkv's workspace, or the share of
 * the keys another device holds) as long as they follow this layout.
 */
int fa_merge_partials(const float* o_parts, const float* lse_parts, int num_parts,
                      int B, int H, int N, int d, int out_dtype, void* o, float* lse,
                      hipStream_t stream);

/*
 * fa_fwd_gqa -- the forward pass with grouped-query attention ("Kernels and
 * Memory in LLM Inference", section "Store less: MQA, GQA, MLA": the query
 * heads are split into groups and each group shares one key head and one
 * value head; Hkv = 1 is multi-query attention, Hkv = Hq ordinary multi-head
 * attention). The groups are runs of consecutive query heads: query head h
 * reads key/value head h / (Hq / Hkv).
 *
 *   q, o       [B, Hq, N, d];  lse [B, Hq, N]  (as fa_fwd with H = Hq).
 *   k, v       [B, Hkv, N, d]; Hq must be a multiple of Hkv (else FA_ERR_SHAPE).
 *   descales   FP8 only: device float [B*Hq + 2*B*Hkv]: q per query head, then
 *              k, then v per key/value head (for Hkv = Hq this is fa_fwd's
 *              [3][B*H]).
 *   num_splits 1 runs the unsplit kernels (workspace ignored, may be NULL);
 *              2..FA_MAX_SPLITS the split-KV path of fa_fwd_splitkv, with a
 *              workspace of fa_splitkv_workspace_bytes(B, Hq, N, d, num_splits)
 *              bytes laid out as there (partials per query head).
 * Everything else as fa_fwd / fa_fwd_splitkv.
 */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int N, int d, int causal, float scale, int dtype,
               const float* descales, int num_splits, void* workspace, size_t workspace_bytes,
               hipStream_t stream);

/*
 * fa_bwd -- the FlashAttention-2 backward pass, bf16 ("FlashAttention-2 from
 * PyTorch to Triton", forward-pass section and its list of what the first
 * kernel leaves out; "Kernels and Memory in LLM Inference", section
 * "Training detour (brief)"). From the forward's inputs, its output O and
 * its L, and the upstream gradient dO, with P = exp(scale Q K^T - L)
 * recomputed tile by tile and D = rowsum(dO * O):
 *   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q.
 * For grouped-query attention a key/value head's dK, dV sum over its group's
 * query heads.
 *
 *   q, o, dout  [B, Hq, N, d] bfloat16 (o: fa_fwd's output for these inputs).
 *   k, v        [B, Hkv, N, d] bfloat16; Hq a multiple of Hkv.
 *   lse         [B, Hq, N] float: fa_fwd's L.
 *   dq          [B, Hq, N, d] bfloat16 output; dk, dv [B, Hkv, N, d].
 *   d           64 or 128.   causal, scale: as in the forward.
 *   dtype       FA_DTYPE_BF16 only (anything else: FA_ERR_DTYPE).
 *   workspace   device memory owned by the caller, 16-byte aligned, at least
 *               fa_bwd_workspace_bytes(B, Hq, N) bytes, that function asked
 *               with the device the call runs on current: per query row the
 *               pair (L log2 e, D) in float, and on grids too small to give
 *               every compute unit two dQ workgroups (B*Hq*ceil(N/128) below
 *               twice the CU count, N >= 2048) the fp32 partial dQ of S key
 *               chunks (S = 2..8, no chunk under 1024 keys). Calls sharing it
 *               must not overlap.
 * Enqueues three kernels (the (L, D) pass, then dK/dV and dQ), and a fourth
 * that sums the dQ partials in chunk order when the keys are chunked. dQ is
 * formed in its own pass over the key tiles, without atomics: the result is
 * deterministic. All tensor pointers 16-byte aligned.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N);
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
           int causal, float scale, int dtype, void* workspace, size_t workspace_bytes,
           hipStream_t stream);

/* Human-readable name of a fa_status_t value. Never NULL. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
