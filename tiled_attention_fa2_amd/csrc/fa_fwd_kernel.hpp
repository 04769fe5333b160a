// FlashAttention-2 forward for gfx950 (MI355X), one kernel template for the
// fp32, bf16 and FP8-e4m3 variants.
//
// What it computes ("FlashAttention-2 from PyTorch to Triton", forward-pass
// section and Triton kernel walkthrough; "1.8x Faster Attention on an RTX
// 5080", sections "The loop starts" through "After the last strip"): for one
// query tile, loop over key tiles in ascending order, form the score tile,
// keep a running row max m and row sum l, rescale the running output by
// exp(m_old - m_new), add P V, and divide by l once at the end; also write
// L = m + log l.
//
// How it maps onto CDNA4:
//   * One workgroup = NWAVES wavefronts of 64 lanes = one (batch*head, query
//     tile of 32*NWAVES rows). Each wave owns 32 query rows to the end: no
//     exchange between waves except the shared K/V tiles in LDS.
//   * Scores are formed transposed, S^T = K Q^T, with the 32x32 MFMA
//     (A = K tile from LDS, B = Q^T held in registers for the whole loop).
//     In the 32x32 accumulator layout lane l holds column l%32 = one query
//     and 16 keys (rows 8j + 4*(l/32) + i), so a row max / row sum is an
//     in-lane reduction plus one exchange between lanes l and l+32
//     (v_permlane32_swap).
//   * The output is formed transposed too, O^T += V^T P^T. P^T is the B
//     operand, and lane l needs query l%32's probabilities: exactly the
//     scores the lane already holds. So P never leaves registers. The MFMA
//     sums over operand slots, not over key indices, so the V^T operand only
//     has to present V rows in the same key order as the P slots. That order
//     is baked into the LDS address where each V element is written (the
//     "key order" idea of "1.8x Faster Attention on an RTX 5080", section
//     "P stays in registers", moved from a prepare pass into the LDS store).
//   * K/V tiles go global -> registers -> LDS, double buffered: the loads for
//     tile j+1 are issued before tile j is computed and written to the other
//     LDS buffer after it, one barrier per tile. V is stored transposed
//     (feature-major) in LDS so every MFMA operand read is one contiguous
//     16- or 32-byte LDS read. Rows are padded by 16 bytes so that eight
//     consecutive rows start in eight different 16-byte bank groups.
//   * exp2 with scale*log2(e) folded into one FMA per score; masking only on
//     tiles that hold keys >= N or straddle the causal diagonal; the causal
//     key loop stops at the diagonal and a wave skips the MFMA work of tiles
//     entirely above its rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum DType { kF32 = 0, kBF16 = 1, kFP8 = 2 };

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Element size, k-slots per lane of one MFMA operand and operand dwords.
//   f32 : v_mfma_f32_32x32x2_f32,        K = 2,  1 value  per lane
//   bf16: v_mfma_f32_32x32x16_bf16,      K = 16, 8 values per lane
//   fp8 : v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, unit scales),
//         K = 64, 32 values per lane
template <int DT> struct Traits;
template <> struct Traits<kF32>  { static constexpr int ES = 4; static constexpr int KPL = 1;  };
template <> struct Traits<kBF16> { static constexpr int ES = 2; static constexpr int KPL = 8;  };
template <> struct Traits<kFP8>  { static constexpr int ES = 1; static constexpr int KPL = 32; };

// Reinterpretation of a 32-bit value. Taking the argument by value matters:
// __builtin_bit_cast applied directly to an element of an ext_vector_type
// value has been seen to read element 0 whatever the index.
__host__ __device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__host__ __device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

template <int DT> struct Operand {
  static constexpr int DW = Traits<DT>::KPL * Traits<DT>::ES / 4;
  uint32_t w[DW];
};

template <int DT>
__device__ __forceinline__ void mfma(const Operand<DT>& a, const Operand<DT>& b, f32x16& c) {
  if constexpr (DT == kBF16) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else if constexpr (DT == kFP8) {
    // format code 0 = e4m3 for both operands; E8M0 scale 127 = 2^0
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a),
                                                        __builtin_bit_cast(i32x8, b), c,
                                                        0, 0, 0, 127, 0, 127);
  } else {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(u2f(a.w[0]), u2f(b.w[0]), c, 0, 0, 0);
  }
}

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* descales;  // [3][BH] for fp8, else unused
  int BH;
  int N;
  int n_qtiles;
  int causal;
  float scale;
};

// Static shape of one instantiation.
template <int DT, int D, int BN, int NWAVES>
struct Cfg {
  static constexpr int ES = Traits<DT>::ES;
  static constexpr int KPL = Traits<DT>::KPL;
  static constexpr int NT = 64 * NWAVES;          // threads per workgroup
  static constexpr int BM = 32 * NWAVES;          // query rows per workgroup
  static constexpr int NB = BN / 32;              // 32-key blocks per tile
  static constexpr int QK_STEPS = D / (2 * KPL);  // MFMAs per 32x32 score block
  static constexpr int PV_STEPS = BN / (2 * KPL); // k-steps of the PV product
  static constexpr int MB = D / 32;               // 32-row blocks of O^T
  static constexpr int KROW = D * ES + 16;        // padded LDS row of K (bytes)
  static constexpr int VROW = BN * ES + 16;       // padded LDS row of V^T (bytes)
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int KCHUNKS = BN * D * ES / 16;            // 16-byte chunks per K tile
  static constexpr int KPT = (KCHUNKS + NT - 1) / NT;         // per thread
  static constexpr int CPR = D * ES / 16;                     // 16-byte chunks per row
  static constexpr int EPC = 16 / ES;                         // elements per chunk
  static constexpr int VITEMS = (BN / 4) * CPR;               // (4-key group, chunk) items
  static constexpr int VPT = (VITEMS + NT - 1) / NT;
  static_assert(BN % 32 == 0, "key tile must be a multiple of 32");
  static_assert(BN % (2 * KPL) == 0, "key tile must cover whole PV k-steps");
  static_assert(D % (2 * KPL) == 0 && D % 32 == 0, "head dim");
  static_assert(KCHUNKS % NT == 0, "K tile must split evenly over the threads");
};

// Position, inside one key tile of V^T in LDS, of key `key` (0 <= key < BN).
// The score of key 32b + 8jj + 4hh + i sits in lane half hh at accumulator
// slot 4jj + i of block b; counting the lane's slots across blocks
// (r = 16b + 4jj + i), PV k-step n takes slots [n*KPL, (n+1)*KPL) from each
// lane half, and the half-hh lanes read their KPL V^T values starting at
// n*2*KPL + hh*KPL. Writing key `key` there makes every V^T operand read one
// contiguous run.
template <int KPL>
__host__ __device__ __forceinline__ constexpr int vt_pos(int key) {
  const int b = key >> 5, jj = (key >> 3) & 3, hh = (key >> 2) & 1, i = key & 3;
  const int r = 16 * b + 4 * jj + i;
  const int n = r / KPL, s = r % KPL;
  return n * 2 * KPL + hh * KPL + s;
}

// Exchange between the two 32-lane halves of a wave: on return, lane l holds
// in (a, b) the entry values of lanes l%32 and l%32 + 32 (v_permlane32_swap
// swaps the upper half of its first operand with the lower half of its
// second). Written as inline asm with two distinct registers: the compiler
// builtin, given the same value twice, has been seen to fold its two results
// into one. The s_nop covers the VALU-write -> permlane-read wait states.
// Must run with the whole wave active.
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float swap_halves_max(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float swap_halves_min(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return fminf(a, b);
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return a + b;
}

// Block index -> logical work item. Workgroups are dispatched round-robin over
// the 8 XCDs; this remap hands every XCD a contiguous range of logical items,
// so the query tiles resident on one XCD share a head and its K/V stream
// through that XCD's L2. Logical items run head by head; within a head, causal
// tiles go longest first.
__host__ __device__ __forceinline__ void work_item(int bid, int total, int n_qtiles, int causal,
                                          int& bh, int& qt) {
  const int per = total >> 3, rem = total & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  const int lin = (xcd < rem) ? xcd * (per + 1) + slot
                              : rem * (per + 1) + (xcd - rem) * per + slot;
  bh = lin / n_qtiles;
  const int t = lin - bh * n_qtiles;
  qt = causal ? (n_qtiles - 1 - t) : t;
}

template <int DT, int D, int BN, int NWAVES, bool CAUSAL>
__global__ void __launch_bounds__(64 * NWAVES)
fa_fwd_kernel(FwdArgs p) {
  using C = Cfg<DT, D, BN, NWAVES>;
  using Op = Operand<DT>;
  constexpr int ES = C::ES, KPL = C::KPL;

  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  int bh, qt;
  work_item(blockIdx.x, p.BH * p.n_qtiles, p.n_qtiles, CAUSAL ? 1 : 0, bh, qt);
  const int N = p.N;
  const int q0 = qt * C::BM;
  const int q0w = q0 + 32 * wave;
  const int my_q = q0w + l32;

  const size_t head_off = (size_t)bh * (size_t)N * D;  // elements
  const unsigned char* Qg = (const unsigned char*)p.q + head_off * ES;
  const unsigned char* Kg = (const unsigned char*)p.k + head_off * ES;
  const unsigned char* Vg = (const unsigned char*)p.v + head_off * ES;

  // scale * log2(e), with the fp8 descales of Q and K folded in
  float c = p.scale * 1.4426950408889634f;
  float pv_scale = 1.0f;
  if constexpr (DT == kFP8) {
    c *= p.descales[bh] * p.descales[p.BH + bh];
    pv_scale = p.descales[2 * p.BH + bh] * (1.0f / 256.0f);
  }
  const bool c_nonneg = c >= 0.0f;
  const float masked_raw = c_nonneg ? -__builtin_inff() : __builtin_inff();

  // ---- Q^T operands, held in registers for the whole loop ----
  Op qop[C::QK_STEPS];
  {
    const bool qvalid = my_q < N;
    const unsigned char* qrow = Qg + (size_t)(qvalid ? my_q : 0) * D * ES;
#pragma unroll
    for (int kk = 0; kk < C::QK_STEPS; ++kk) {
      const unsigned char* src = qrow + (size_t)(kk * 2 * KPL + hh * KPL) * ES;
#pragma unroll
      for (int w = 0; w < Op::DW; ++w)
        qop[kk].w[w] = qvalid ? ((const uint32_t*)src)[w] : 0u;
    }
  }

  // ---- key-tile range ----
  int n_ktiles = (N + BN - 1) / BN;
  if constexpr (CAUSAL) {
    const int last = (q0 + C::BM - 1) / BN + 1;
    n_ktiles = n_ktiles < last ? n_ktiles : last;
  }

  // ---- staging registers for the next K / V tile ----
  u32x4 kst[C::KPT];
  u32x4 vst[C::VPT][4];

  auto load_tile = [&](int j) {
    const int kbase = j * BN;
#pragma unroll
    for (int it = 0; it < C::KPT; ++it) {
      const int ch = tid + it * C::NT;
      const int row = ch / C::CPR, cc = ch % C::CPR;
      const int key = kbase + row;
      kst[it] = (key < N) ? *(const u32x4*)(Kg + ((size_t)key * D * ES + cc * 16))
                          : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
      const int item = tid + it * C::NT;
      if (C::VITEMS % C::NT == 0 || item < C::VITEMS) {
        const int g = item % (BN / 4), cc = item / (BN / 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kbase + 4 * g + i;
          vst[it][i] = (key < N) ? *(const u32x4*)(Vg + ((size_t)key * D * ES + cc * 16))
                                 : u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    unsigned char* Ks = smem + buf * C::STAGE;
    unsigned char* Vs = Ks + C::KBYTES;
#pragma unroll
    for (int it = 0; it < C::KPT; ++it) {
      const int ch = tid + it * C::NT;
      const int row = ch / C::CPR, cc = ch % C::CPR;
      *(u32x4*)(Ks + row * C::KROW + cc * 16) = kst[it];
    }
#pragma unroll
    for (int it = 0; it < C::VPT; ++it) {
      const int item = tid + it * C::NT;
      if (C::VITEMS % C::NT == 0 || item < C::VITEMS) {
        const int g = item % (BN / 4), cc = item / (BN / 4);
        // four consecutive keys land at four consecutive positions for bf16
        // and fp8; fp32 positions are two apart
        const int pos0 = vt_pos<KPL>(4 * g);
#pragma unroll
        for (int e = 0; e < C::EPC; ++e) {
          const int dcol = cc * C::EPC + e;
          unsigned char* dst = Vs + dcol * C::VROW;
          if constexpr (ES == 2) {
            const int w = e >> 1, sh = (e & 1) * 16;
            const uint32_t a0 = (vst[it][0][w] >> sh) & 0xffffu;
            const uint32_t a1 = (vst[it][1][w] >> sh) & 0xffffu;
            const uint32_t a2 = (vst[it][2][w] >> sh) & 0xffffu;
            const uint32_t a3 = (vst[it][3][w] >> sh) & 0xffffu;
            uint2 pk;
            pk.x = a0 | (a1 << 16);
            pk.y = a2 | (a3 << 16);
            *(uint2*)(dst + pos0 * 2) = pk;
          } else if constexpr (ES == 1) {
            const int w = e >> 2, sh = (e & 3) * 8;
            const uint32_t a0 = (vst[it][0][w] >> sh) & 0xffu;
            const uint32_t a1 = (vst[it][1][w] >> sh) & 0xffu;
            const uint32_t a2 = (vst[it][2][w] >> sh) & 0xffu;
            const uint32_t a3 = (vst[it][3][w] >> sh) & 0xffu;
            *(uint32_t*)(dst + pos0) = a0 | (a1 << 8) | (a2 << 16) | (a3 << 24);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              *(uint32_t*)(dst + vt_pos<KPL>(4 * g + i) * 4) = vst[it][i][e];
          }
        }
      }
    }
  };

  // ---- running state: O^T accumulators, m (scaled, log2 units), lane-partial l ----
  f32x16 oacc[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[mb][r] = 0.0f;
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_ktiles; ++j) {
    const int buf = j & 1;
    const bool has_next = j + 1 < n_ktiles;
    if (has_next) load_tile(j + 1);

    const int kbase = j * BN;
    // a wave whose 32 rows all lie above this tile's first key skips it
    const bool wave_active = !CAUSAL || kbase <= q0w + 31;
    if (wave_active) {
      const unsigned char* Ks = smem + buf * C::STAGE;
      const unsigned char* Vs = Ks + C::KBYTES;

      // S^T = K Q^T, one 32x32 block per 32 keys
      f32x16 s[C::NB];
#pragma unroll
      for (int b = 0; b < C::NB; ++b) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[b][r] = 0.0f;
        const unsigned char* krow = Ks + (32 * b + l32) * C::KROW + hh * KPL * ES;
#pragma unroll
        for (int kk = 0; kk < C::QK_STEPS; ++kk) {
          Op a;
          const uint32_t* src = (const uint32_t*)(krow + kk * 2 * KPL * ES);
#pragma unroll
          for (int w = 0; w < Op::DW; ++w) a.w[w] = src[w];
          mfma<DT>(a, qop[kk], s[b]);
        }
      }

      // masking, only on tiles that hold keys >= N or cross the diagonal
      const bool need_mask = (kbase + BN > N) || (CAUSAL && kbase + BN - 1 > q0w);
      if (need_mask) {
#pragma unroll
        for (int b = 0; b < C::NB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kbase + 32 * b + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool ok = key < N && (!CAUSAL || key <= my_q);
            s[b][r] = ok ? s[b][r] : masked_raw;
          }
      }

      // row extreme of the raw scores (max when c >= 0, min when c < 0)
      float ext;
      if (c_nonneg) {
        ext = s[0][0];
#pragma unroll
        for (int b = 0; b < C::NB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) ext = fmaxf(ext, s[b][r]);
        ext = swap_halves_max(ext);
      } else {
        ext = s[0][0];
#pragma unroll
        for (int b = 0; b < C::NB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) ext = fminf(ext, s[b][r]);
        ext = swap_halves_min(ext);
      }
      // every processed (row, tile) pair holds at least one valid key, so ext
      // is finite and so is m_new
      const float m_new = fmaxf(m_run, ext * c);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;

      // p = exp2(s*c - m_new); masked keys give 0
      float psum = 0.0f;
#pragma unroll
      for (int b = 0; b < C::NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float t = __builtin_fmaf(s[b][r], c, -m_new);
          if (need_mask) {
            const int key = kbase + 32 * b + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool ok = key < N && (!CAUSAL || key <= my_q);
            t = ok ? t : -__builtin_inff();
          }
          const float pv = __builtin_amdgcn_exp2f(t);
          s[b][r] = pv;
          psum += pv;
        }
      l_run = alpha * l_run + psum;

      // O^T *= alpha (skipped when the max did not move for any row of the wave)
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
      }

      // P^T operands, straight from the score registers
      Op pop[C::PV_STEPS];
#pragma unroll
      for (int n = 0; n < C::PV_STEPS; ++n) {
        if constexpr (DT == kBF16) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int r0 = n * KPL + 2 * w;
            const float x0 = s[r0 >> 4][r0 & 15], x1 = s[(r0 + 1) >> 4][(r0 + 1) & 15];
            const __bf16 b0 = (__bf16)x0, b1 = (__bf16)x1;
            pop[n].w[w] = (uint32_t)__builtin_bit_cast(unsigned short, b0) |
                          ((uint32_t)__builtin_bit_cast(unsigned short, b1) << 16);
          }
        } else if constexpr (DT == kFP8) {
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const int r0 = n * KPL + 4 * w;
            int v = 0;
            v = __builtin_amdgcn_cvt_pk_fp8_f32(s[r0 >> 4][r0 & 15] * 256.0f,
                                                s[(r0 + 1) >> 4][(r0 + 1) & 15] * 256.0f, v, false);
            v = __builtin_amdgcn_cvt_pk_fp8_f32(s[(r0 + 2) >> 4][(r0 + 2) & 15] * 256.0f,
                                                s[(r0 + 3) >> 4][(r0 + 3) & 15] * 256.0f, v, true);
            pop[n].w[w] = (uint32_t)v;
          }
        } else {
          const int r0 = n;
          pop[n].w[0] = f2u(s[r0 >> 4][r0 & 15]);
        }
      }

      // O^T += V^T P^T
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const unsigned char* vrow = Vs + (32 * mb + l32) * C::VROW + hh * KPL * ES;
#pragma unroll
        for (int n = 0; n < C::PV_STEPS; ++n) {
          Op a;
          const uint32_t* src = (const uint32_t*)(vrow + n * 2 * KPL * ES);
#pragma unroll
          for (int w = 0; w < Op::DW; ++w) a.w[w] = src[w];
          mfma<DT>(a, pop[n], oacc[mb]);
        }
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: full row sum, L, O / l, bounded stores ----
  const float l_tot = swap_halves_sum(l_run);
  const float inv = pv_scale / l_tot;
  if (my_q < N) {
    if (hh == 0)
      p.lse[(size_t)bh * N + my_q] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.6931471805599453f;
    const size_t obase = ((size_t)bh * N + my_q) * D;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * mb + 8 * jj + 4 * hh;
        const float x0 = oacc[mb][4 * jj + 0] * inv, x1 = oacc[mb][4 * jj + 1] * inv;
        const float x2 = oacc[mb][4 * jj + 2] * inv, x3 = oacc[mb][4 * jj + 3] * inv;
        if constexpr (DT == kF32) {
          *(float4*)((float*)p.o + obase + d0) = make_float4(x0, x1, x2, x3);
        } else {
          const __bf16 b0 = (__bf16)x0, b1 = (__bf16)x1, b2 = (__bf16)x2, b3 = (__bf16)x3;
          uint2 pk;
          pk.x = (uint32_t)__builtin_bit_cast(unsigned short, b0) |
                 ((uint32_t)__builtin_bit_cast(unsigned short, b1) << 16);
          pk.y = (uint32_t)__builtin_bit_cast(unsigned short, b2) |
                 ((uint32_t)__builtin_bit_cast(unsigned short, b3) << 16);
          *(uint2*)((unsigned short*)p.o + obase + d0) = pk;
        }
      }
  }
}

}  // namespace fa
