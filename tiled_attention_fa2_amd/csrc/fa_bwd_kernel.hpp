// FlashAttention-2 backward for gfx950 (MI355X): bf16, head dim 64 or 128.
//
// What it computes ("FlashAttention-2 from PyTorch to Triton", forward-pass
// section and its list of what the first kernel leaves out; "Kernels and
// Memory in LLM Inference", section "Training detour (brief)"): the forward
// stored L = m + log l per row, so every tile of P is recomputed on chip as
// P = exp(S - L) instead of being kept; with D = rowsum(dO * O) per row,
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//     dQ = scale dS K,  dK = scale dS^T Q.
// Three kernels:
//   fa_bwd_pre_kernel    D per row and L in log2 units, into the workspace;
//   fa_bwd_dkdv_kernel   one workgroup per (key/value head, 128 keys): every
//                        wave keeps its 32 keys' K and V rows as MFMA
//                        operands and its dK, dV accumulators, and streams the
//                        query tiles (Q, dO and the (L, D) pairs) of every
//                        query head of its group through LDS;
//   fa_bwd_dq_kernel     one workgroup per (query head, 128 queries), the
//                        "second pass" for dQ: every wave keeps its 32 query
//                        rows of Q and dO and its dQ accumulator and streams
//                        the K/V tiles, so no atomics are needed and the
//                        result is deterministic.
//
// How it maps onto CDNA4 (the layouts of the forward kernel, roles swapped
// where needed):
//   * dK/dV kernel: S = Q K^T with A = Q rows from LDS and B = the wave's K
//     rows; the 32x32 accumulator gives lane l key l%32 and 16 queries, so P
//     and dS are B operands as they stand for dV^T += dO^T P and
//     dK^T += Q^T dS, whose A operands (dO^T, Q^T) come from the Q / dO tiles
//     with the LDS transpose read ds_read_b64_tr_b16, in the query order of
//     the register slots (the forward's V^T read with keys and queries
//     swapped). dP = dO V^T has the same layout as S.
//   * dQ kernel: S^T = K Q^T and dP^T = V dO^T (A = K, V rows from LDS;
//     B = the wave's Q, dO rows), P^T and dS^T per lane, and
//     dQ^T += K^T dS^T with K^T read transposed from the K tile: the forward
//     kernel with one more product and no running max (L is known).
//   * Tiles go global -> LDS by DMA (buffer_load ... lds issued from inline
//     asm, as in the forward), two stages, rows XOR-swizzled per 16-byte
//     chunk with (row & 7); the transposed reads use the same swizzle.
//   * Masking (keys or queries >= N, causal key > query) only on tiles that
//     need it: masked scores give p = 0 whatever the sign of the scale.
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa {

struct BwdArgs {
  const void* q;        // [BH][N][D] bf16
  const void* k;        // [BH / group][N][D]
  const void* v;        // [BH / group][N][D]
  const void* o;        // [BH][N][D] forward output
  const void* dout;     // [BH][N][D] upstream gradient dO
  const float* lse;     // [BH][N] natural-log L of the forward
  float2* ld;           // workspace [BH][N]: (L * log2 e, D)
  void* dq;             // [BH][N][D] bf16 outputs
  void* dk;             // [BH / group][N][D]
  void* dv;             // [BH / group][N][D]
  int BH;               // batch * query heads
  int N;
  int group;            // query heads per key/value head
  int n_tiles;          // 128-row tiles per head (dQ kernel)
  int n_ktiles;         // key tiles per head of the dK/dV kernel (128 KB keys each)
  int causal_order;     // order of the dQ kernel's causal tiles (work_item)
  int causal_order_kv;  // order of the dK/dV kernel's causal key blocks (work_item, flipped)
  float scale;
  // dQ key split (kernels instantiated with SPLIT): chunk s of a query tile
  // takes the 32-key tiles [s * dq_chunk_tiles, (s + 1) * dq_chunk_tiles) and
  // writes its unscaled fp32 partial dQ to dq_part[s]; fa_bwd_dq_merge_kernel
  // sums the parts in order.
  int dq_splits;
  int dq_chunk_tiles;
  float* dq_part;       // [dq_splits][BH][N][D] fp32
};

// D = rowsum(dO * O) in fp32 and L in log2 units, one row per D/8 lanes.
template <int D>
__global__ void __launch_bounds__(256) fa_bwd_pre_kernel(BwdArgs p) {
  constexpr int TPR = D / 8;          // lanes per row, 8 bf16 (16 bytes) each
  constexpr int RPB = 256 / TPR;
  const long long rows = (long long)p.BH * p.N;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.0f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)((const unsigned short*)p.o + row * D + 8 * c);
    const u32x4 b = *(const u32x4*)((const unsigned short*)p.dout + row * D + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = a[i], y = b[i];
      acc += u2f(x << 16) * u2f(y << 16);
      acc += u2f(x & 0xffff0000u) * u2f(y & 0xffff0000u);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && c == 0) p.ld[row] = make_float2(p.lse[row] * 1.4426950408889634f, acc);
}

namespace bwd {

constexpr int kNWaves = 4;
constexpr int kRows = 32 * kNWaves;   // rows of the fixed side per workgroup

// Shapes shared by both kernels: a streamed tile has 32 rows of D bf16.
template <int D>
struct Shape {
  static constexpr int ES = 2, KPL = 8;
  static constexpr int ROW = D * ES;                  // bytes per row
  static constexpr int CPR = ROW / 16;                // 16-byte chunks per row
  static constexpr int TILE = 32 * ROW;               // bytes per 32-row tile
  static constexpr int NINSTR = TILE / 1024 / kNWaves;
  static constexpr int T_ROWS = 64 * kNWaves / CPR;   // rows between DMA instructions
  static constexpr int QK_STEPS = D / (2 * KPL);      // MFMAs over D
  static constexpr int PV_STEPS = 32 / (2 * KPL);     // MFMAs over the 32 streamed rows
  static constexpr int MB = D / 32;
  static_assert(TILE % (1024 * kNWaves) == 0, "tile must split into whole DMA instructions");
  static_assert(CPR >= 8, "swizzle needs at least 8 chunks per row");
  static_assert(T_ROWS % 8 == 0, "swizzle period");
};

// Per-lane bases of the two LDS read patterns of a 32-row tile swizzled with
// (row & 7): row-major A operands (lane = row, 16 bytes of k) and transposed
// A operands (ds_read_b64_tr_b16: lane = feature, keys/queries in the order of
// the 32x32 accumulator's register slots).
template <int D>
struct ReadBases {
  uint32_t rm[4];   // row-major: read at rm[kk & 3] + 128 (kk >> 2)
  uint32_t tr[2];   // transposed: read at tr[mb & 1] + 128 (mb >> 1) + (16 n + 8 t) ROW
  __device__ __forceinline__ ReadBases(int lane) {
    using S = Shape<D>;
    const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int u = 0; u < 4; ++u) rm[u] = (uint32_t)l32 * S::ROW + 16 * ((2 * u + hh) ^ (l32 & 7));
    const int vg = lane >> 4, vj = lane & 15, va = vg & 1;
    const int e = vj >> 2, q = vj & 3, r0 = 4 * hh + e, x = 2 * va + (q >> 1);
#pragma unroll
    for (int m1 = 0; m1 < 2; ++m1)
      tr[m1] = (uint32_t)r0 * S::ROW + 16 * ((4 * m1 + x) ^ (r0 & 7)) + 8 * (q & 1);
  }
};

template <int D>
__device__ __forceinline__ void read_rm(const unsigned char* tile, const ReadBases<D>& rb, int kk,
                                        Operand<kBF16>& a) {
  const u32x4 w = *(const u32x4*)(tile + rb.rm[kk & 3] + 128 * (kk >> 2));
#pragma unroll
  for (int y = 0; y < 4; ++y) a.w[y] = w[y];
}

template <int D>
__device__ __forceinline__ void read_tr(const unsigned char* tile, const ReadBases<D>& rb, int mb, int n,
                                        Operand<kBF16>& a) {
  using S = Shape<D>;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const unsigned char* src = tile + rb.tr[mb & 1] + 128 * (mb >> 1) + (16 * n + 8 * t) * S::ROW;
    const s16x4_t v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)src);
    const i32x2_t v2 = __builtin_bit_cast(i32x2_t, v4);
    a.w[2 * t] = (uint32_t)v2[0];
    a.w[2 * t + 1] = (uint32_t)v2[1];
  }
}

// Scheduling order of a phase of STEPS steps, each R LDS reads feeding M
// MFMAs: the reads of the first LOOK steps, then the MFMAs of one step and the
// reads LOOK steps ahead, and so on. At one wave per SIMD nothing else hides an
// LDS read's latency, and left to itself the compiler issues each step's reads
// right before the MFMAs that need them.
template <int STEPS, int R, int M, int LOOK>
__device__ __forceinline__ void pipeline_reads() {
  static_assert(LOOK >= 1 && LOOK < STEPS, "look-ahead inside the phase");
  __builtin_amdgcn_sched_group_barrier(0x100, LOOK * R, 0);
#pragma unroll
  for (int i = 0; i < STEPS - LOOK; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, LOOK * M, 0);
}

// S and dP of the dK/dV kernel as inline-asm MFMAs, so that their
// accumulators are VGPRs. The compiler gives all MFMAs of a kernel one register
// class; with the dK/dV accumulators taking every AGPR it chose AGPRs for S and
// dP as well, then copied them out for the softmax and moved dK/dV accumulators
// to VGPRs and back to make room, every tile. Hidden in asm, these MFMAs carry
// their own wait states: two before (a VALU write of an operand, e.g. a copy
// the compiler adds) and drain_vacc() before the VALU reads the results.
template <bool FIRST>
__device__ __forceinline__ void mfma_vacc(const Operand<kBF16>& a, const Operand<kBF16>& b, f32x16& c) {
  const u32x4 av = {a.w[0], a.w[1], a.w[2], a.w[3]};
  const u32x4 bv = {b.w[0], b.w[1], b.w[2], b.w[3]};
  if constexpr (FIRST)
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(av), "v"(bv));
  else
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(av), "v"(bv));
}
// 16 wait states: an 8-pass MFMA's result is readable by other instructions
// after 12 on gfx950.
template <int KB>
__device__ __forceinline__ void drain_vacc(f32x16 (&s)[KB], f32x16 (&dp)[KB]) {
  static_assert(KB == 1 || KB == 2, "one or two key blocks");
  if constexpr (KB == 1)
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(dp[0]));
  else
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]), "+v"(dp[0]), "+v"(dp[1]));
}

// One 32-row tile of a [N][D] bf16 head (rows from r_first; rows >= N read as
// zero) into LDS at `lds` by DMA: every wave issues NINSTR instructions under
// one descriptor, instruction t at the lane offsets goff + t T_ROWS ROW.
template <int D>
__device__ __forceinline__ void dma_tile(const unsigned char* head, int N, int r_first, uint32_t lds,
                                         int wave, uint32_t goff) {
  using S = Shape<D>;
  const int rem = N - r_first;
  const i32x4_t r = dma_rsrc(head + (size_t)(rem > 0 ? r_first : N) * S::ROW, rem > 0 ? (uint32_t)rem * S::ROW : 0u);
#pragma unroll
  for (int t = 0; t < S::NINSTR; ++t) {
    const uint32_t l = lds + 1024 * (wave + kNWaves * t);
    if (t == 0)
      lds_dma16_rsrc<4>(r, l, goff);
    else
      lds_dma16_rsrc<0>(r, l, goff + (uint32_t)(t * S::T_ROWS * S::ROW));
  }
}

// Packs 16 fp32 accumulator values of one lane into the bf16 B operands of
// the PV-shaped products, in the slot order the transposed reads assume.
__device__ __forceinline__ void pack_b(const float (&x)[16], Operand<kBF16> (&op)[2]) {
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int w = 0; w < 4; ++w) op[n].w[w] = pack_bf16(x[n * 8 + 2 * w], x[n * 8 + 2 * w + 1]);
}

// 32 rows x D of a lane's accumulators (lane = row l32, 16 values per 32
// features) -> bf16 row `row` of `out`, times `mul`.
template <int MB>
__device__ __forceinline__ void store_rows(void* out, size_t row, int hh, const f32x16 (&acc)[MB],
                                           float mul) {
  constexpr int D = 32 * MB;
  unsigned short* dst = (unsigned short*)out + row * D;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d0 = 32 * mb + 8 * jj + 4 * hh;
      uint2 pk;
      pk.x = pack_bf16(acc[mb][4 * jj + 0] * mul, acc[mb][4 * jj + 1] * mul);
      pk.y = pack_bf16(acc[mb][4 * jj + 2] * mul, acc[mb][4 * jj + 3] * mul);
      *(uint2*)(dst + d0) = pk;
    }
}

}  // namespace bwd

// ---------------------------------------------------------------------------
#ifndef FA_DQ_LOOK
#define FA_DQ_LOOK 2
#endif
constexpr int kDqLook = FA_DQ_LOOK;   // MFMA steps of LDS reads in flight

// dQ: one workgroup per (batch * query head, 128 queries); waves own 32 rows.
// SPLIT: one workgroup per (batch * query head, 128 queries, key chunk), for
// grids that would otherwise leave the SIMDs with fewer than two waves ("Kernels
// and Memory in LLM Inference", section "Flash-Decoding: one token, whole
// chip": the keys cut into chunks whose partial results are summed after).
template <int D, bool CAUSAL, bool SPLIT = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa_bwd_dq_kernel(BwdArgs p) {
  using S = bwd::Shape<D>;
  using Op = Operand<kBF16>;
  constexpr int QK = S::QK_STEPS, PV = S::PV_STEPS, MB = S::MB, ROW = S::ROW, TILE = S::TILE;
  constexpr int STAGE = 2 * TILE;    // K tile, V tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  int bh, qt, sp = 0;
  if constexpr (SPLIT) {
    int t;
    work_item(blockIdx.x, p.BH * p.n_tiles * p.dq_splits, p.n_tiles * p.dq_splits, CAUSAL ? p.causal_order : 0,
              bh, t);
    qt = t / p.dq_splits;
    sp = t - qt * p.dq_splits;
  } else {
    work_item(blockIdx.x, p.BH * p.n_tiles, p.n_tiles, CAUSAL ? p.causal_order : 0, bh, qt);
  }
  const int N = p.N;
  const int q0 = qt * bwd::kRows;
  const int q0w = q0 + 32 * wave;
  const int my_q = q0w + l32;
  const uint32_t head_bytes = (uint32_t)N * ROW;
  const int bkv = bh / p.group;
  const unsigned char* Qg = (const unsigned char*)p.q + (size_t)bh * head_bytes;
  const unsigned char* dOg = (const unsigned char*)p.dout + (size_t)bh * head_bytes;
  const unsigned char* Kg = (const unsigned char*)p.k + (size_t)bkv * head_bytes;
  const unsigned char* Vg = (const unsigned char*)p.v + (size_t)bkv * head_bytes;
  const float c = p.scale * 1.4426950408889634f;

  // the wave's Q and dO rows: B operands of S^T = K Q^T and dP^T = V dO^T
  Op qop[QK], dop[QK];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qg, head_bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dOg, head_bytes);
    const uint32_t off = (uint32_t)my_q * ROW + hh * 16;
#pragma unroll
    for (int kk = 0; kk < QK; ++kk) {
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rq, off + kk * 32, 0, 0);
      const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rd, off + kk * 32, 0, 0);
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        qop[kk].w[y] = a[y];
        dop[kk].w[y] = b[y];
      }
    }
  }
  const float2 ld = my_q < N ? p.ld[(size_t)bh * N + my_q] : make_float2(0.0f, 0.0f);

  int T = (N + 31) / 32;
  if constexpr (CAUSAL) {
    const int last = (q0 + bwd::kRows - 1) / 32 + 1;
    T = T < last ? T : last;
  }
  int j_begin = 0, j_end = T;
  if constexpr (SPLIT) {
    j_begin = sp * p.dq_chunk_tiles;
    j_end = j_begin + p.dq_chunk_tiles < T ? j_begin + p.dq_chunk_tiles : T;
  }

  const int dma_row = (64 * wave + lane) / S::CPR;
  const int dma_pc = lane % S::CPR;
  const uint32_t goff = (uint32_t)dma_row * ROW + 16 * (dma_pc ^ (dma_row & 7));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_ptr)smem;
  auto issue = [&](int jt, int buf) {
    const uint32_t st = lds0 + buf * STAGE;
    bwd::dma_tile<D>(Kg, N, jt * 32, st, wave, goff);
    bwd::dma_tile<D>(Vg, N, jt * 32, st + TILE, wave, goff);
  };
  const bwd::ReadBases<D> rb(lane);

  f32x16 dq[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[mb][r] = 0.0f;

  if (j_begin < j_end) issue(j_begin, j_begin & 1);
  wait_vmcnt<0>();
  __syncthreads();
  for (int j = j_begin; j < j_end; ++j) {
    const int buf = j & 1;
    if (j + 1 < j_end) issue(j + 1, buf ^ 1);
    const int kbase = j * 32;
    const bool wave_active = !CAUSAL || kbase <= q0w + 31;
    if (wave_active) {
      const unsigned char* st = smem + buf * STAGE;
      f32x16 s, dpt;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.0f;
        dpt[r] = 0.0f;
      }
#pragma unroll
      for (int kk = 0; kk < QK; ++kk) {
        Op a, b;
        bwd::read_rm<D>(st, rb, kk, a);
        mfma<kBF16>(a, qop[kk], s);
        bwd::read_rm<D>(st + TILE, rb, kk, b);
        mfma<kBF16>(b, dop[kk], dpt);
      }
      bwd::pipeline_reads<QK, 2, 2, kDqLook>();
      // P^T = exp2(S^T c - L2), dS^T = P^T (dP^T - D); key kbase + 4hh + rel
      const bool need_mask = (kbase + 32 > N) || (CAUSAL && kbase + 31 > q0w);
      float ds[16];
      if (__builtin_expect(need_mask, 0)) {   // rare: its code out of line
        asm volatile("" ::: "memory");
        int lim = N - kbase - 4 * hh;
        if constexpr (CAUSAL) {
          const int lim_c = my_q - kbase - 4 * hh + 1;
          lim = lim < lim_c ? lim : lim_c;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = 8 * (r >> 2) + (r & 3);
          const float t = rel < lim ? __builtin_fmaf(s[r], c, -ld.x) : -__builtin_inff();
          const float pr = __builtin_amdgcn_exp2f(t);
          ds[r] = pr * (dpt[r] - ld.y);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -ld.x));
          ds[r] = pr * (dpt[r] - ld.y);
        }
      }
      Op dsop[2];
      bwd::pack_b(ds, dsop);
      // dQ^T += K^T dS^T (K^T read transposed from the K tile)
#pragma unroll
      for (int n = 0; n < PV; ++n)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          Op a;
          bwd::read_tr<D>(st, rb, mb, n, a);
          mfma<kBF16>(a, dsop[n], dq[mb]);
        }
      bwd::pipeline_reads<PV * MB, 2, 1, kDqLook>();
    }
    wait_vmcnt<0>();
    __syncthreads();
  }
  if (my_q < N) {
    if constexpr (SPLIT) {
      // the chunk's unscaled partial, zero where the chunk has no tile
      float* dst = p.dq_part + (((size_t)sp * p.BH + bh) * (size_t)N + my_q) * D;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d0 = 32 * mb + 8 * jj + 4 * hh;
          *(float4*)(dst + d0) = make_float4(dq[mb][4 * jj + 0], dq[mb][4 * jj + 1], dq[mb][4 * jj + 2],
                                             dq[mb][4 * jj + 3]);
        }
    } else {
      bwd::store_rows<MB>(p.dq, (size_t)bh * N + my_q, hh, dq, p.scale);
    }
  }
}

// dQ of the key split: scale * (part 0 + part 1 + ...), summed in chunk order
// (deterministic), to bf16. One row of D values per D/8 lanes, 8 each.
template <int D>
__global__ void __launch_bounds__(256) fa_bwd_dq_merge_kernel(BwdArgs p) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const long long rows = (long long)p.BH * p.N;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= rows) return;
  const int c0 = 8 * (threadIdx.x % TPR);
  const size_t stride = (size_t)rows * D;
  const float* src = p.dq_part + (size_t)row * D + c0;
  float4 a = *(const float4*)src, b = *(const float4*)(src + 4);
  for (int s = 1; s < p.dq_splits; ++s) {
    const float4 x = *(const float4*)(src + s * stride), y = *(const float4*)(src + s * stride + 4);
    a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
    b.x += y.x; b.y += y.y; b.z += y.z; b.w += y.w;
  }
  const float m = p.scale;
  uint4 pk;
  pk.x = pack_bf16(a.x * m, a.y * m);
  pk.y = pack_bf16(a.z * m, a.w * m);
  pk.z = pack_bf16(b.x * m, b.y * m);
  pk.w = pack_bf16(b.z * m, b.w * m);
  *(uint4*)((unsigned short*)p.dq + (size_t)row * D + c0) = pk;
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (batch * key/value head, 128 KB keys); each wave
// owns KB blocks of 32 keys and loops over the query tiles of every query head
// of its group. The kernel waits on its LDS reads: at one wave per SIMD with
// every register taken, nothing else hides a read's latency, so every MFMA
// phase reads its operands two steps ahead of the MFMAs that use them, and
// with KB = 2 every Q / dO operand read, row-major or transposed, feeds the
// MFMAs of both key blocks, which halves the read-and-wait rounds per flop. The K and V operands of
// blocks b < KREG stay in registers; those of the others (when registers do not
// suffice) in LDS, lane-major per operand, each lane reading back only what it
// wrote (16 cheap row-major reads per tile and block, no bank conflicts).
// The dK/dV accumulators (KB = 2: all 256 AGPRs) are the only MFMA
// accumulators in AGPRs: S and dP come from asm MFMAs into VGPRs (mfma_vacc),
// where the softmax reads them without copies.
#ifndef FA_DKDV_LOOK
#define FA_DKDV_LOOK 2
#endif
constexpr int kDkdvLook = FA_DKDV_LOOK;   // MFMA steps of LDS reads in flight

template <int D, bool CAUSAL, int KB, int KREG>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
fa_bwd_dkdv_kernel(BwdArgs p) {
  using S = bwd::Shape<D>;
  using Op = Operand<kBF16>;
  constexpr int QK = S::QK_STEPS, MB = S::MB, ROW = S::ROW, TILE = S::TILE;
  static_assert(S::PV_STEPS == 2, "two contraction steps over a 32-query tile: the softmax halves");
  constexpr int STAGE = 2 * TILE + 1024;    // Q tile, dO tile, 32 (L2, D) pairs (1 KB slot)
  static_assert(KREG >= 1 && KREG <= KB, "at least one key block in registers");
  constexpr int KVL_WAVE = (KB - KREG) * 2 * QK * 1024;   // staged K, V operands of one wave
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE + bwd::kNWaves * KVL_WAVE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  const int BHkv = p.BH / p.group;
  int bkv, kt;
  // causal: key block 0 meets every query tile and the last block the fewest,
  // so the longest items are the first blocks; work_item hands out its last
  // tiles first, hence the flip (a bijection either way)
  work_item(blockIdx.x, BHkv * p.n_ktiles, p.n_ktiles, CAUSAL ? p.causal_order_kv : 0, bkv, kt);
  if constexpr (CAUSAL) kt = p.n_ktiles - 1 - kt;
  const int N = p.N;
  const int k0 = kt * bwd::kRows * KB;
  const int k0w = k0 + 32 * KB * wave;      // the wave's first key; block b: k0w + 32 b
  const uint32_t head_bytes = (uint32_t)N * ROW;
  const unsigned char* Kg = (const unsigned char*)p.k + (size_t)bkv * head_bytes;
  const unsigned char* Vg = (const unsigned char*)p.v + (size_t)bkv * head_bytes;
  const float c = p.scale * 1.4426950408889634f;

  // the wave's K and V rows: B operands of S = Q K^T and dP = dO V^T; blocks
  // b >= KREG go to the wave's LDS region: operand (b, K or V, kk) of lane l at
  // ((b - KREG) * 2 QK + (K: 0, V: QK) + kk) * 1024 + 16 l
  Op kop[KREG][QK], vop[KREG][QK];
  unsigned char* kvl = smem + 2 * STAGE + wave * KVL_WAVE;
  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg, head_bytes);
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const uint32_t off = (uint32_t)(k0w + 32 * b + l32) * ROW + hh * 16;
#pragma unroll
      for (int kk = 0; kk < QK; ++kk) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rk, off + kk * 32, 0, 0);
        const u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(rv, off + kk * 32, 0, 0);
        if (b < KREG) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            kop[b < KREG ? b : 0][kk].w[w] = x[w];
            vop[b < KREG ? b : 0][kk].w[w] = y[w];
          }
        } else {
          unsigned char* dst = kvl + ((b - KREG) * 2 * QK + kk) * 1024 + 16 * lane;
          *(u32x4*)dst = x;
          *(u32x4*)(dst + QK * 1024) = y;
        }
      }
    }
  }

  const int dma_row = (64 * wave + lane) / S::CPR;
  const int dma_pc = lane % S::CPR;
  const uint32_t goff = (uint32_t)dma_row * ROW + 16 * (dma_pc ^ (dma_row & 7));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_ptr)smem;
  const bwd::ReadBases<D> rb(lane);

  f32x16 dk[KB][MB], dv[KB][MB];
#pragma unroll
  for (int b = 0; b < KB; ++b)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[b][mb][r] = 0.0f;
        dv[b][mb][r] = 0.0f;
      }

  const int T = (N + 31) / 32;
  // causal: queries before the workgroup's first key see none of its keys
  const int j_first = CAUSAL ? k0 / 32 : 0;
  for (int g = 0; g < p.group; ++g) {
    const int bh = bkv * p.group + g;
    const unsigned char* Qg = (const unsigned char*)p.q + (size_t)bh * head_bytes;
    const unsigned char* dOg = (const unsigned char*)p.dout + (size_t)bh * head_bytes;
    const float2* LDg = p.ld + (size_t)bh * N;
    auto issue = [&](int jt, int buf) {
      const uint32_t st = lds0 + buf * STAGE;
      bwd::dma_tile<D>(Qg, N, jt * 32, st, wave, goff);
      bwd::dma_tile<D>(dOg, N, jt * 32, st + TILE, wave, goff);
      if (wave == 0) {
        // lanes 0-15 bring the tile's 32 (L2, D) pairs, the rest read zeros or
        // the next tile's pairs into the unused part of the 1 KB slot
        const int q = jt * 32;
        const uint32_t bytes = q < N ? (uint32_t)(N - q) * 8u : 0u;
        lds_dma16(LDg + (q < N ? q : N), bytes, st + 2 * TILE, (uint32_t)lane * 16u);
      }
    };
    if (j_first < T) issue(j_first, 0);
    wait_vmcnt<0>();
    __syncthreads();
    for (int j = j_first; j < T; ++j) {
      const int buf = (j - j_first) & 1;
      if (j + 1 < T) issue(j + 1, buf ^ 1);
      const int qbase = j * 32;
      // causal: a tile entirely before the wave's first key contributes nothing
      const bool wave_active = !CAUSAL || qbase + 31 >= k0w;
      if (wave_active) {
        const unsigned char* st = smem + buf * STAGE;
        f32x16 s[KB], dp[KB];
        // the operands of step kk: Q and dO rows, and the K, V operands of the
        // blocks staged in LDS; read kDkdvLook steps ahead of their MFMAs (the
        // scheduler's MFMA groups do not see asm, so the order is written out,
        // one scheduling fence per step)
        constexpr int NL = KB - KREG > 0 ? KB - KREG : 1;
        struct StepOps { Op a, bo, kl[NL], vl[NL]; };
        StepOps ops[kDkdvLook + 1];
        auto load_step = [&](int kk, StepOps& o) {
          bwd::read_rm<D>(st, rb, kk, o.a);
          bwd::read_rm<D>(st + TILE, rb, kk, o.bo);
#pragma unroll
          for (int b = KREG; b < KB; ++b) {
            const u32x4 x = *(const u32x4*)(kvl + ((b - KREG) * 2 * QK + kk) * 1024 + 16 * lane);
            const u32x4 y = *(const u32x4*)(kvl + ((b - KREG) * 2 * QK + QK + kk) * 1024 + 16 * lane);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              o.kl[b - KREG].w[w] = x[w];
              o.vl[b - KREG].w[w] = y[w];
            }
          }
        };
#pragma unroll
        for (int kk = 0; kk < kDkdvLook; ++kk) load_step(kk, ops[kk]);
#pragma unroll
        for (int kk = 0; kk < QK; ++kk) {
          const StepOps& o = ops[kk % (kDkdvLook + 1)];
#pragma unroll
          for (int b = 0; b < KB; ++b) {
            const Op& kb_op = b < KREG ? kop[b < KREG ? b : 0][kk] : o.kl[b >= KREG ? b - KREG : 0];
            if (kk == 0) bwd::mfma_vacc<true>(o.a, kb_op, s[b]);
            else bwd::mfma_vacc<false>(o.a, kb_op, s[b]);
          }
#pragma unroll
          for (int b = 0; b < KB; ++b) {
            const Op& vb_op = b < KREG ? vop[b < KREG ? b : 0][kk] : o.vl[b >= KREG ? b - KREG : 0];
            if (kk == 0) bwd::mfma_vacc<true>(o.bo, vb_op, dp[b]);
            else bwd::mfma_vacc<false>(o.bo, vb_op, dp[b]);
          }
          if (kk + kDkdvLook < QK) load_step(kk + kDkdvLook, ops[(kk + kDkdvLook) % (kDkdvLook + 1)]);
          __builtin_amdgcn_sched_barrier(0);
        }
        bwd::drain_vacc<KB>(s, dp);
        // (L2, D) of the lane's 16 queries qbase + 8 (r / 4) + 4 hh + r % 4
        float l2[16], dd[16];
        const float* ldt = (const float*)(st + 2 * TILE);
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          const int q4 = 8 * b4 + 4 * hh;
          const float4 x0 = *(const float4*)(ldt + 2 * q4);
          const float4 x1 = *(const float4*)(ldt + 2 * q4 + 4);
          l2[4 * b4 + 0] = x0.x; dd[4 * b4 + 0] = x0.y;
          l2[4 * b4 + 1] = x0.z; dd[4 * b4 + 1] = x0.w;
          l2[4 * b4 + 2] = x1.x; dd[4 * b4 + 2] = x1.y;
          l2[4 * b4 + 3] = x1.z; dd[4 * b4 + 3] = x1.w;
        }
        // P = exp2(S c - L2), dS = P (dP - D), in two halves of the lane's
        // 16 slots: slots 8h .. 8h + 7 make the operands of contraction step
        // n = h of the products below, so the products of step 0 need only
        // half 0 and half 1 can be computed beside them. Query qbase + 4hh +
        // rel is valid for key block b iff it is < N and (causal) >= the
        // lane's key; invalid slots are computed like the others, then set to
        // zero (a masked slot's exp2 may overflow; the select drops it).
        const bool need_mask = (qbase + 32 > N) || (CAUSAL && qbase < k0w + 32 * KB - 1);
        Op pop[KB][2], dsop[KB][2];
        float pv[KB][8], ds[KB][8];
        auto soft = [&](int h) {
#pragma unroll
          for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int r = 8 * h + i;
              pv[b][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], c, -l2[r]));
              ds[b][i] = pv[b][i] * (dp[b][r] - dd[r]);
            }
        };
        auto fix_and_pack = [&](int h) {
          if (__builtin_expect(need_mask, 0)) {   // rare: its code out of line
            asm volatile("" ::: "memory");
            const int hi = N - qbase - 4 * hh;   // rel < hi
#pragma unroll
            for (int b = 0; b < KB; ++b) {
              const int lo = CAUSAL ? k0w + 32 * b + l32 - qbase - 4 * hh : -(1 << 30);   // rel >= lo
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                const int r = 8 * h + i;
                const int rel = 8 * (r >> 2) + (r & 3);
                const bool ok = rel < hi && rel >= lo;
                pv[b][i] = ok ? pv[b][i] : 0.0f;
                ds[b][i] = ok ? ds[b][i] : 0.0f;
              }
            }
          }
#pragma unroll
          for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              pop[b][h].w[w] = pack_bf16(pv[b][2 * w], pv[b][2 * w + 1]);
              dsop[b][h].w[w] = pack_bf16(ds[b][2 * w], ds[b][2 * w + 1]);
            }
        };
        // dV^T += dO^T P and dK^T += Q^T dS for contraction step n (A operands
        // read transposed, once for all key blocks)
        auto products = [&](int n) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            Op a, bq;
            bwd::read_tr<D>(st + TILE, rb, mb, n, a);
#pragma unroll
            for (int b = 0; b < KB; ++b) mfma<kBF16>(a, pop[b][n], dv[b][mb]);
            bwd::read_tr<D>(st, rb, mb, n, bq);
#pragma unroll
            for (int b = 0; b < KB; ++b) mfma<kBF16>(bq, dsop[b][n], dk[b][mb]);
          }
        };
        constexpr int LKH = kDkdvLook < MB ? kDkdvLook : MB - 1;   // look-ahead inside a half
        soft(0);
        fix_and_pack(0);
        products(0);
        soft(1);
        bwd::pipeline_reads<MB, 4, 2 * KB, LKH>();
        fix_and_pack(1);
        products(1);
        bwd::pipeline_reads<MB, 4, 2 * KB, LKH>();
      }
      wait_vmcnt<0>();
      __syncthreads();
    }
  }
#pragma unroll
  for (int b = 0; b < KB; ++b) {
    const int my_k = k0w + 32 * b + l32;
    if (my_k < N) {
      const size_t row = (size_t)bkv * N + my_k;
      bwd::store_rows<MB>(p.dk, row, hh, dk[b], p.scale);
      bwd::store_rows<MB>(p.dv, row, hh, dv[b], 1.0f);
    }
  }
}

}  // namespace fa
