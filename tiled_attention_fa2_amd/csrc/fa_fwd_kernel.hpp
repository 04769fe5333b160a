// FlashAttention-2 forward for gfx950 (MI355X): fa_fwd_kernel (fp32, K/V
// staged through registers) and fa_fwd_dma_kernel (bf16 and FP8-e4m3, K/V
// fetched into LDS by DMA, further below).
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
//   * fa_fwd_kernel: K/V tiles go global -> registers -> LDS, double
//     buffered: the loads for tile j+1 are issued before tile j is computed
//     and written to the other LDS buffer after it, one barrier per tile. V
//     is stored transposed (feature-major) in LDS so every MFMA operand read
//     is one contiguous LDS read. Rows are padded by 16 bytes so that eight
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

// The fp8 MFMA with per-block scales. In this instruction lane half h, slot s
// of an operand holds contraction index k = 32 (s / 16) + 16 h + s % 16, so
// block b (k = 32b .. 32b + 31) is slots 16b .. 16b + 15 of both lane halves,
// and its E8M0 scale for row i of A (column j of B) is byte OPA (OPB) of the
// scale register of lane i + 32b (j + 32b).
template <int OPA, int OPB>
__device__ __forceinline__ void mfma_fp8_scaled(const Operand<kFP8>& a, const Operand<kFP8>& b,
                                                f32x16& c, int scale_a, int scale_b) {
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a),
                                                      __builtin_bit_cast(i32x8, b), c,
                                                      0, 0, OPA, scale_a, OPB, scale_b);
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
  // Order of causal work items (work_item): 1 = head by head, 2 = longest
  // query tiles first across the heads each XCD holds. Chosen by the host.
  int causal_order;
  float scale;
  // Split-KV mode (kernels instantiated with SPLIT): split s of a query tile
  // takes the keys [s * split_keys, (s + 1) * split_keys) and writes its
  // partial result to o_part / lse_part instead of o / lse.
  int n_splits;
  int split_keys;     // a multiple of 128
  float* o_part;      // [n_splits][BH][N][D] fp32
  float* lse_part;    // [n_splits][BH][N] fp32
  // Grouped-query attention ("Kernels and Memory in LLM Inference", section
  // "Store less: MQA, GQA, MLA"): `group` consecutive query heads share one
  // key/value head, so (batch*query head) bh reads K/V head bh / group of the
  // BH / group key/value heads. group = 1 is ordinary multi-head attention.
  // FP8 descales: q at [bh], k at [BH + bh / group], v at [BH + BH / group + bh / group].
  int group;
  // Per-block FP8 (kernels instantiated with MX): E8M0 scales, one byte
  // (exponent + 127) per block of 32 elements along each product's
  // contraction axis. q_scale [BH][N][D/32], k_scale [BH/group][N][D/32],
  // v_scale [BH/group][ceil(N/32)][D].
  const unsigned char* q_scale;
  const unsigned char* k_scale;
  const unsigned char* v_scale;
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
  static constexpr int ROW = D * ES;              // bytes of one Q/K/V row in memory
  static constexpr int KROW = ROW + 16;           // padded LDS row of K (bytes)
  static constexpr int VROW = BN * ES + 16;       // padded LDS row of V^T (bytes)
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int CPR = ROW / 16;                        // 16-byte chunks per row
  static constexpr int KCHUNKS = BN * CPR;                    // 16-byte chunks per K tile
  static constexpr int KPT = (KCHUNKS + NT - 1) / NT;         // per thread (rounded up)
  static constexpr int EPC = 16 / ES;                         // elements per chunk
  static constexpr int VITEMS = (BN / 4) * CPR;               // (4-key group, chunk) items
  static constexpr int VPT = (VITEMS + NT - 1) / NT;
  static_assert(BN % 32 == 0, "key tile must be a multiple of 32");
  static_assert(BN % (2 * KPL) == 0, "key tile must cover whole PV k-steps");
  static_assert(D % (2 * KPL) == 0 && D % 32 == 0, "head dim");
  static_assert(KCHUNKS % NT == 0 || KCHUNKS < NT, "K tile chunks must split evenly");
  static_assert(VITEMS % 64 == 0, "V items must fill whole waves");
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
// Maximum / minimum that propagate NaN (llvm.maximum / llvm.minimum): on gfx950
// they map to v_maximum3_f32 / v_minimum3_f32 as they stand. fmaxf / fminf
// (IEEE maxNum) would make the compiler quiet every MFMA output with an extra
// v_max_f32 first, doubling the cost of a row maximum. Scores are never NaN for
// finite inputs (masked ones are -inf), so the two agree on every valid input.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmin(float a, float b) { return __builtin_elementwise_minimum(a, b); }

__device__ __forceinline__ float swap_halves_max(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return vmax(a, b);
}
__device__ __forceinline__ float swap_halves_min(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return vmin(a, b);
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
// tiles go longest first (causal = 1). With causal = 2 and whole heads per
// XCD (heads a multiple of 8), the XCD's items go longest first across all of
// its heads (the longest tile of every head, then the next, ...), so no long
// tile of a late head starts while the rest of the XCD is draining; the host
// picks it when those heads' K/V are small enough to share the caches.
__host__ __device__ __forceinline__ void work_item(int bid, int total, int n_qtiles, int causal,
                                          int& bh, int& qt) {
  const int per = total >> 3, rem = total & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  if (causal == 2 && rem == 0 && per % n_qtiles == 0) {
    const int heads = per / n_qtiles;
    const int rank = slot / heads;   // 0: the longest tile
    bh = xcd * heads + (slot - rank * heads);
    qt = n_qtiles - 1 - rank;
    return;
  }
  const int lin = (xcd < rem) ? xcd * (per + 1) + slot
                              : rem * (per + 1) + (xcd - rem) * per + slot;
  bh = lin / n_qtiles;
  const int t = lin - bh * n_qtiles;
  qt = causal ? (n_qtiles - 1 - t) : t;
}

// Work item of a workgroup and its key-tile range [j_begin, j_end) out of the
// n_ktiles tiles its query tile needs. Split-KV: the split index runs fastest
// within a query tile, and split s takes the tiles holding the keys
// [s * split_keys, (s + 1) * split_keys) ("Kernels and Memory in LLM
// Inference", section "Flash-Decoding: one token, whole chip": the keys are cut
// into chunks, one workgroup per chunk).
template <bool SPLIT, int BN>
__device__ __forceinline__ void split_item(const FwdArgs& p, int causal, int& bh, int& qt, int& sp) {
  if constexpr (SPLIT) {
    int t;
    work_item(blockIdx.x, p.BH * p.n_qtiles * p.n_splits, p.n_qtiles * p.n_splits, causal, bh, t);
    qt = t / p.n_splits;
    sp = t - qt * p.n_splits;
  } else {
    work_item(blockIdx.x, p.BH * p.n_qtiles, p.n_qtiles, causal, bh, qt);
    sp = 0;
  }
}
template <bool SPLIT, int BN>
__device__ __forceinline__ void key_tile_range(const FwdArgs& p, int sp, int n_ktiles, int& j_begin,
                                               int& j_end) {
  if constexpr (SPLIT) {
    const int per = p.split_keys / BN;
    j_begin = sp * per;
    j_end = j_begin + per < n_ktiles ? j_begin + per : n_ktiles;
  } else {
    j_begin = 0;
    j_end = n_ktiles;
  }
}

// Split-KV epilogue of one lane: the chunk's output divided by the chunk's own
// sum, in fp32, and the chunk's natural-log logsumexp L = ln2 (m2 + log2 l)
// (m2 = running max in log2 units, bias removed). A row with no valid key in
// the chunk (l = 0) gets O = 0 and L = -inf.
template <int MB>
__device__ __forceinline__ void store_partial(const FwdArgs& p, int sp, int bh, int my_q, int hh,
                                              const f32x16 (&oacc)[MB], float l_tot, float m2,
                                              float dv) {
  constexpr int D = 32 * MB;
  if (my_q >= p.N) return;
  const size_t prow = ((size_t)sp * p.BH + bh) * (size_t)p.N + my_q;
  const bool empty = !(l_tot > 0.0f);
  const float inv = empty ? 0.0f : dv / l_tot;
  if (hh == 0)
    p.lse_part[prow] = empty ? -__builtin_inff() : (m2 + __builtin_amdgcn_logf(l_tot)) * 0.6931471805599453f;
  float* dst = p.o_part + prow * D;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d0 = 32 * mb + 8 * jj + 4 * hh;
      *(float4*)(dst + d0) = make_float4(oacc[mb][4 * jj + 0] * inv, oacc[mb][4 * jj + 1] * inv,
                                         oacc[mb][4 * jj + 2] * inv, oacc[mb][4 * jj + 3] * inv);
    }
}

// Pairwise reduction of n values (n a power of two): depth log2(n) instead of
// a chain of n - 1 dependent operations.
template <int NV, typename Get, typename Op2>
__device__ __forceinline__ float tree_reduce(Get get, Op2 op) {
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = get(i);
#pragma unroll
  for (int w = NV / 2; w >= 1; w /= 2)
#pragma unroll
    for (int i = 0; i < w; ++i) v[i] = op(v[i], v[i + w]);
  return v[0];
}

template <bool B> struct BoolTag { static constexpr bool value = B; };

// Scheduling pattern for a run of NMFMA MFMAs whose A operands come from LDS
// (RPM ds_reads per MFMA): LOOK operands are read ahead, then each MFMA is
// followed by the reads of a later operand. Without it the scheduler hoists
// every read of the run to its top and runs out of registers.
template <int NMFMA, int RPM, int LOOK>
__device__ __forceinline__ void interleave_reads_with_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, LOOK * RPM, 0);
#pragma unroll
  for (int i = 0; i < NMFMA - LOOK; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, LOOK, 0);
}

// Max of n values (n a multiple of 8) as four interleaved chains of
// three-input maxima (v_maximum3_f32): about n/2 instructions, short chains.
template <int NV, typename Get>
__device__ __forceinline__ float max_reduce(Get get) {
  static_assert(NV % 8 == 0, "max_reduce takes a multiple of 8 values");
  float m0 = vmax(get(0), get(1)), m1 = vmax(get(2), get(3));
  float m2 = vmax(get(4), get(5)), m3 = vmax(get(6), get(7));
#pragma unroll
  for (int i = 8; i < NV; i += 8) {
    m0 = vmax(vmax(m0, get(i + 0)), get(i + 1));
    m1 = vmax(vmax(m1, get(i + 2)), get(i + 3));
    m2 = vmax(vmax(m2, get(i + 4)), get(i + 5));
    m3 = vmax(vmax(m3, get(i + 6)), get(i + 7));
  }
  return vmax(vmax(m0, m1), vmax(m2, m3));
}

// Buffer resource over [base, base + bytes): loads at offsets >= bytes return
// zero, which is how rows past the end of a head read as zeros without a
// branch. 0x00020000 is the gfx9 raw-buffer word 3 (32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}


typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two floats -> one dword of two bf16 (round to nearest even), low half first
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// WPE = waves per SIMD the register allocation must allow (1 or 2): with 2,
// two workgroups share a CU and one wave's softmax overlaps another's MFMAs.
// LOOK > 0 pins the order of each run of MFMAs and their LDS operand reads,
// with LOOK operands read ahead (0 leaves the order to the compiler).
// The fp32 forward (true fp32 MFMA, v_mfma_f32_32x32x2_f32), any head dim the
// host accepts (64, 128).
template <int DT, int D, int BN, int NWAVES, bool CAUSAL, int WPE, int LOOK = 0, bool SPLIT = false>
__global__ void __launch_bounds__(64 * NWAVES) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
fa_fwd_kernel(FwdArgs p) {
  static_assert(DT == kF32, "register-staged kernel: fp32 (bf16 and FP8 run fa_fwd_dma_kernel)");
  using C = Cfg<DT, D, BN, NWAVES>;
  using Op = Operand<DT>;
  constexpr int ES = C::ES, KPL = C::KPL;

  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  int bh, qt, sp;
  split_item<SPLIT, BN>(p, CAUSAL ? p.causal_order : 0, bh, qt, sp);
  const int N = p.N;
  const int q0 = qt * C::BM;
  const int q0w = q0 + 32 * wave;
  const int my_q = q0w + l32;

  const uint32_t head_bytes = (uint32_t)N * C::ROW;   // < 2^31, checked by the host
  const int bkv = bh / p.group;                       // key/value head
  const size_t head_off = (size_t)bh * head_bytes;
  const size_t kv_off = (size_t)bkv * head_bytes;
  const unsigned char* Qg = (const unsigned char*)p.q + head_off;
  const unsigned char* Kg = (const unsigned char*)p.k + kv_off;
  const unsigned char* Vg = (const unsigned char*)p.v + kv_off;

  // scale * log2(e)
  float c = p.scale * 1.4426950408889634f;
  // scale == 0: every valid score gets the same weight. A tiny positive c
  // gives exactly that (|s * c| < 2^-24, so exp2 rounds to 1) and lets a
  // masked score be -inf rather than -inf * 0 = NaN.
  if (c == 0.0f) c = 1e-30f;
  const bool c_pos = c > 0.0f;
  const float masked_raw = c_pos ? -__builtin_inff() : __builtin_inff();

  // ---- Q^T operands, held in registers for the whole loop ----
  Op qop[C::QK_STEPS];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qg, head_bytes);
    // rows >= N start at or past head_bytes and read as zero
    const uint32_t qoff = (uint32_t)my_q * C::ROW + hh * KPL * ES;
#pragma unroll
    for (int kk = 0; kk < C::QK_STEPS; ++kk) {
      const uint32_t off = qoff + kk * 2 * KPL * ES;
      if constexpr (Op::DW >= 4) {
#pragma unroll
        for (int x = 0; x < Op::DW / 4; ++x) {
          const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16 * x, 0, 0);
#pragma unroll
          for (int y = 0; y < 4; ++y) qop[kk].w[4 * x + y] = w[y];
        }
      } else {
        qop[kk].w[0] = __builtin_amdgcn_raw_buffer_load_b32(rq, off, 0, 0);
      }
    }
  }

  // ---- key-tile range ----
  int n_ktiles = (N + BN - 1) / BN;
  if constexpr (CAUSAL) {
    const int last = (q0 + C::BM - 1) / BN + 1;
    n_ktiles = n_ktiles < last ? n_ktiles : last;
  }
  int j_begin, j_end;
  key_tile_range<SPLIT, BN>(p, sp, n_ktiles, j_begin, j_end);

  // ---- per-lane constant offsets ----
  // K staging: chunk tid + it*NT of the tile -> row, 16-byte column
  const int k_row0 = tid / C::CPR, k_col = tid % C::CPR;
  const uint32_t k_goff = (uint32_t)k_row0 * C::ROW + k_col * 16;
  const uint32_t k_soff = (uint32_t)k_row0 * C::KROW + k_col * 16;
  constexpr int K_ROWS_PER_IT = C::NT / C::CPR;
  // V staging: item tid -> 4-key group g, 16-byte column cc (waves past the
  // last item skip the V work)
  constexpr int V_WAVES = C::VITEMS < C::NT ? C::VITEMS / 64 : NWAVES;
  const bool v_worker = wave < V_WAVES;
  const int v_g = tid % (BN / 4), v_cc = tid / (BN / 4);
  const uint32_t v_goff = (uint32_t)(4 * v_g) * C::ROW + v_cc * 16;
  const uint32_t v_soff = C::KBYTES + (uint32_t)(v_cc * C::EPC) * C::VROW +
                          (uint32_t)vt_pos<KPL>(4 * v_g) * ES;
  // MFMA operand reads
  const uint32_t k_roff = (uint32_t)l32 * C::KROW + hh * KPL * ES;
  const uint32_t v_roff = C::KBYTES + (uint32_t)l32 * C::VROW + hh * KPL * ES;

  u32x4 kst[C::KPT];
  u32x4 vst[C::VPT][4];

  auto load_tile = [&](int j) {
    const uint32_t kbase = (uint32_t)j * BN;
    const uint32_t rem = head_bytes - kbase * C::ROW;     // bytes from this tile to the end
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg + (size_t)kbase * C::ROW, rem);
#pragma unroll
    for (int it = 0; it < C::KPT; ++it)
      kst[it] = __builtin_amdgcn_raw_buffer_load_b128(rk, k_goff + it * K_ROWS_PER_IT * C::ROW, 0, 0);
    if (v_worker) {
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg + (size_t)kbase * C::ROW, rem);
#pragma unroll
      for (int it = 0; it < C::VPT; ++it)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vst[it][i] = __builtin_amdgcn_raw_buffer_load_b128(
              rv, v_goff + it * (C::NT / (BN / 4)) * 16 + i * C::ROW, 0, 0);
    }
  };

  auto store_tile = [&](int buf) {
    unsigned char* st = smem + buf * C::STAGE;
#pragma unroll
    for (int it = 0; it < C::KPT; ++it)
      *(u32x4*)(st + k_soff + it * K_ROWS_PER_IT * C::KROW) = kst[it];
    if (v_worker) {
#pragma unroll
      for (int it = 0; it < C::VPT; ++it) {
        unsigned char* dst0 = st + v_soff + it * (C::NT / (BN / 4)) * C::EPC * C::VROW;
        // four keys land two positions apart
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *(uint32_t*)(dst0 + e * C::VROW + (vt_pos<KPL>(4 * v_g + i) - vt_pos<KPL>(4 * v_g)) * 4) =
                vst[it][i][e];
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

  if (j_begin < j_end) {
    load_tile(j_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int j = j_begin; j < j_end; ++j) {
    const int buf = (j - j_begin) & 1;
    const bool has_next = j + 1 < j_end;
    if (has_next) load_tile(j + 1);

    const int kbase = j * BN;
    // a wave whose 32 rows all lie above this tile's first key skips it
    const bool wave_active = !CAUSAL || kbase <= q0w + 31;
    if (wave_active) {
      const unsigned char* st = smem + buf * C::STAGE;

      // S^T = K Q^T, one 32x32 block per 32 keys; the blocks alternate so that
      // consecutive MFMAs never wait on each other's accumulator
      f32x16 s[C::NB];
#pragma unroll
      for (int b = 0; b < C::NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[b][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < C::QK_STEPS; ++kk)
#pragma unroll
        for (int b = 0; b < C::NB; ++b) {
          Op a;
          const uint32_t* src = (const uint32_t*)(st + k_roff + b * 32 * C::KROW + kk * 2 * KPL * ES);
#pragma unroll
          for (int w = 0; w < Op::DW; ++w) a.w[w] = src[w];
          mfma<DT>(a, qop[kk], s[b]);
        }
      if constexpr (LOOK > 0)
        interleave_reads_with_mfma<C::QK_STEPS * C::NB, (Op::DW >= 4 ? Op::DW / 4 : 1), LOOK>();

      // Masking, only on tiles that hold keys >= N or cross the diagonal: a
      // masked score becomes -inf after scaling (c != 0 here), so it drops out
      // of the max and exp2 turns it into p = 0. Key kbase + 4hh + rel (rel =
      // 32b + 8jj + i, a compile-time constant per register) is valid iff
      // rel < lim. The empty asm keeps this a real branch: otherwise the
      // compiler turns it into selects that run on every tile.
      const bool need_mask = (kbase + BN > N) || (CAUSAL && kbase + BN - 1 > q0w);
      if (need_mask) {
        asm volatile("" ::: "memory");
        int lim = N - kbase - 4 * hh;
        if constexpr (CAUSAL) {
          const int lim_c = my_q - kbase - 4 * hh + 1;
          lim = lim < lim_c ? lim : lim_c;
        }
#pragma unroll
        for (int b = 0; b < C::NB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rel = 32 * b + 8 * (r >> 2) + (r & 3);
            s[b][r] = rel < lim ? s[b][r] : masked_raw;
          }
      }

      // row extreme of the raw scores (max when c > 0, min when c < 0)
      float ext;
      if (c_pos) {
        ext = max_reduce<C::NB * 16>([&](int i) { return s[i >> 4][i & 15]; });
        ext = swap_halves_max(ext);
      } else {
        ext = -max_reduce<C::NB * 16>([&](int i) { return -s[i >> 4][i & 15]; });
        ext = swap_halves_min(ext);
      }
      // every processed (row, tile) pair holds at least one valid key, so
      // m_tile is finite
      const float m_tile = ext * c;
      const float m_new = m_tile > m_run ? m_tile : m_run;
      // a causal chunk can start above a row's diagonal: until the row meets a
      // valid key its max stays -inf, and a zero reference keeps p = 0, alpha = 0
      float m_ref = m_new;
      if constexpr (SPLIT && CAUSAL) m_ref = m_new == -__builtin_inff() ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
      m_run = m_new;

      // p = exp2(s*c - m_ref)
#pragma unroll
      for (int b = 0; b < C::NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[b][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], c, -m_ref));
      const float psum = tree_reduce<C::NB * 16>([&](int i) { return s[i >> 4][i & 15]; },
                                                 [](float x, float y) { return x + y; });
      l_run = alpha * l_run + psum;

      // O^T *= alpha (skipped when the reference did not move for any row of the wave)
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
      }

      // P^T operands, straight from the score registers
      Op pop[C::PV_STEPS];
#pragma unroll
      for (int n = 0; n < C::PV_STEPS; ++n) pop[n].w[0] = f2u(s[n >> 4][n & 15]);

      // O^T += V^T P^T, the d-blocks alternating between consecutive MFMAs
#pragma unroll
      for (int n = 0; n < C::PV_STEPS; ++n) {
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
          Op a;
          const uint32_t* src =
              (const uint32_t*)(st + v_roff + mb * 32 * C::VROW + n * 2 * KPL * ES);
#pragma unroll
          for (int w = 0; w < Op::DW; ++w) a.w[w] = src[w];
          mfma<DT>(a, pop[n], oacc[mb]);
        }
      }
      if constexpr (LOOK > 0)
        interleave_reads_with_mfma<C::PV_STEPS * C::MB, (Op::DW >= 4 ? Op::DW / 4 : 1), LOOK>();
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: full row sum, L, O / l, bounded stores ----
  const float l_tot = swap_halves_sum(l_run);
  if constexpr (SPLIT) {
    store_partial<C::MB>(p, sp, bh, my_q, hh, oacc, l_tot, m_run, 1.0f);
    return;
  }
  const float inv = 1.0f / l_tot;
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
        *(float4*)((float*)p.o + obase + d0) = make_float4(x0, x1, x2, x3);
      }
  }
}


// ---------------------------------------------------------------------------
// DMA variant (bf16 and fp8, head dim 64 and 128): K and V tiles go global -> LDS
// with buffer_load ... lds (no registers, no LDS store instructions, no
// repacking), row-major with a 16-byte XOR swizzle per row, and the V^T MFMA
// operands are read with the LDS transpose reads:
//   ds_read_b64_tr_b16: in each 16-lane group, lane i element e (e < 4) is
//     element i%4 of the 8 bytes addressed by lane 4e + i/4, i.e. the group
//     reads 4 rows x 16 columns and every lane gets one column;
//   ds_read_b64_tr_b8: lane i byte e (e < 8) is byte i%8 of lane 2e + i/8's
//     8 bytes: 8 rows x 16 columns, one column per lane.
// Each transpose read therefore hands a lane 4 (bf16) or 8 (fp8) keys of one
// feature, and the rows are chosen so that those keys are the ones the lane's
// P^T slots hold (the same key order as vt_pos).
// Swizzles (physical 16-byte chunk = logical chunk ^ f(row)), for the 64
// banks of 4 bytes that serve a 128-bit read 16 lanes at a time and a 64-bit
// read 32 lanes at a time:
//   K, d = 128: f = row & 7  -> the 8 rows an MFMA row-read touches at once
//                               land in 8 different bank groups (16 rows per
//                               phase still meet twice);
//   K, d = 64: bf16 f = (row >> 1) & 7 (two 128-byte rows per bank sweep),
//              fp8 f = (row >> 2) & 3 (four 64-byte rows): the 16 rows of a
//              phase fill all 16 bank groups;
//   V bf16: f = 2 (row & 3)  -> the 4 rows x 32 bytes of a tr16 group hit
//                               8 different bank groups (at d = 64 the whole
//                               32-lane phase is conflict-free);
//   V fp8, d = 128: f = (row & 3) | ((row >> 3) & 1) << 2 -> the same for
//                               tr8's 8 rows x 16 bytes;
//   V fp8, d = 64: f = 2 ((row >> 3) & 1) (four chunks per row).
// Each f depends on row bits 0-3 only, so rows 16 apart share it.
template <int DT, int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D == 128) return row & 7;
  else if constexpr (DT == kBF16) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
template <int DT, int D>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (DT == kBF16) return 2 * (row & 3);
  else if constexpr (D == 128) return (row & 3) | (((row >> 3) & 1) << 2);
  else return 2 * ((row >> 3) & 1);
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Buffer descriptor (wave-uniform SGPRs) of the raw bytes [base, base + bytes):
// loads past its end return zeros.
__device__ __forceinline__ i32x4_t dma_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}
// One LDS DMA instruction: lane L's 16 bytes at byte voff of descriptor r's
// buffer land at LDS address lds + 16 L (lds wave-uniform).
// Written as inline asm on purpose: the compiler tracks a buffer_load ... lds
// it emits itself as an LDS write and, unable to tell the stages of the ring
// apart, waits for every DMA in flight (vmcnt(0)) before the next LDS read,
// i.e. for the prefetch of a later tile before the current one is used. Hidden
// from it, the DMAs are ordered only by the kernel's own wait_vmcnt + barrier
// (extra VMEM operations the compiler does not know of can only make its own
// vmcnt waits stricter). The M0 write needs one wait state before the DMA;
// NOP = 4 gives the five a VMEM read needs after a VALU write of r's SGPRs
// (the readfirstlanes of dma_rsrc), for the first use of a fresh descriptor.
template <int NOP>
__device__ __forceinline__ void lds_dma16_rsrc(const i32x4_t& r, uint32_t lds, uint32_t voff) {
  static_assert(NOP == 0 || NOP == 4, "s_nop 0 or 4");
  const int m0 = __builtin_amdgcn_readfirstlane((int)lds);
  if constexpr (NOP == 4)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(r)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(r)
                 : "memory", "m0");
}
// The same with a descriptor of its own for [base, base + bytes).
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t bytes, uint32_t lds, uint32_t voff) {
  lds_dma16_rsrc<4>(dma_rsrc(base, bytes), lds, voff);
}
// The same with 4 bytes per lane: lane L's dword at byte voff lands at LDS
// address lds + 4 L (a dword past the end of the buffer reads as zero).
__device__ __forceinline__ void lds_dma4(const void* base, uint32_t bytes, uint32_t lds, uint32_t voff) {
  const uint64_t a = (uint64_t)base;
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  const int m0 = __builtin_amdgcn_readfirstlane((int)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(r)
               : "memory", "m0");
}
#pragma clang diagnostic pop

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;
typedef __attribute__((address_space(3))) i32x2_t* lds_i32x2_ptr;
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14, the
// export and LDS counters left at their maxima).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// NSTAGE LDS stages: tile j lives in stage j % NSTAGE and is fetched
// NSTAGE - 1 tiles ahead. WPE = waves per SIMD the registers must allow.
// MX: per-block FP8 (E8M0 scales applied by the MFMAs, see FwdArgs).
// LATE_DMA: the prefetch of each iteration is issued after the tile's QK
// MFMAs instead of before them, so the K reads and MFMAs start right after
// the barrier; the fetch then has one QK phase less to land, which a
// three-stage ring absorbs and a two-stage one does not on long rows.
template <int DT, int BN, int NWAVES, bool CAUSAL, int LOOK, int WPE = 2, int NSTAGE = 2,
          bool SPLIT = false, bool MX = false, int TAUQ = 0, bool LATE_DMA = false, int D = 128>
__global__ void __launch_bounds__(64 * NWAVES) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
fa_fwd_dma_kernel(FwdArgs p) {
  static_assert(DT == kBF16 || DT == kFP8, "DMA variant: bf16 and fp8");
  static_assert(D == 128 || (D == 64 && !MX), "head dim 128, or 64 without per-block scales");
  using Op = Operand<DT>;
  constexpr int ES = Traits<DT>::ES, KPL = Traits<DT>::KPL;
  constexpr int BM = 32 * NWAVES;
  constexpr int NB = BN / 32, QK_STEPS = D / (2 * KPL), PV_STEPS = BN / (2 * KPL), MB = D / 32;
  constexpr int ROW = D * ES, CPR = ROW / 16;
  constexpr int TILE = BN * ROW;                 // bytes of one K or V tile
  // MX: the tile's K scales (BN keys x D/32) and V scales (BN/32 key blocks x
  // D), one dword per lane of one DMA instruction each
  constexpr int SC_K = MX ? BN * (D / 32) : 0;
  constexpr int SC_V = MX ? (BN / 32) * D : 0;
  static_assert(!MX || (DT == kFP8 && NSTAGE == 2 && SC_K == 256 && SC_V == 256),
                "per-block scales: fp8, two stages, one 64-lane dword DMA per scale tile");
  constexpr int STAGE = 2 * TILE + SC_K + SC_V;  // K tile, V tile, then the scales
  constexpr int NINSTR = TILE / 1024 / NWAVES;   // 1 KB DMA instructions per wave per tile
  static_assert(TILE % (1024 * NWAVES) == 0, "tile must split into whole DMA instructions");
  static_assert(CPR >= 4, "swizzles need at least 4 chunks per row");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[NSTAGE * STAGE];
  static_assert(NSTAGE == 2 || NSTAGE == 3, "two or three stages");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  int bh, qt, sp;
  split_item<SPLIT, BN>(p, CAUSAL ? p.causal_order : 0, bh, qt, sp);
  const int N = p.N;
  const int q0 = qt * BM;
  const int q0w = q0 + 32 * wave;
  const int my_q = q0w + l32;

  const uint32_t head_bytes = (uint32_t)N * ROW;
  const int bkv = bh / p.group;                       // key/value head
  const size_t head_off = (size_t)bh * head_bytes;
  const size_t kv_off = (size_t)bkv * head_bytes;
  const unsigned char* Qg = (const unsigned char*)p.q + head_off;
  const unsigned char* Kg = (const unsigned char*)p.k + kv_off;
  const unsigned char* Vg = (const unsigned char*)p.v + kv_off;

  float c = p.scale * 1.4426950408889634f;
  float dv = 1.0f;
  if constexpr (DT == kFP8 && !MX) {
    c *= p.descales[bh] * p.descales[p.BH + bkv];
    dv = p.descales[p.BH + p.BH / p.group + bkv];
  }
  constexpr float kPBias = DT == kFP8 ? 8.0f : 0.0f;
  // Conditional rescale ("Kernels and Memory in LLM Inference", section
  // "FlashAttention-4"): the reference max that p, l and O are taken against
  // moves only when a tile's max exceeds it by more than tau = TAUQ / 4 (log2
  // units); between moves p <= 2^tau (times the bias) and neither O nor l is
  // rescaled, and the tile skips the alpha work. l and O always share the
  // reference, so only the rounding of P changes: with tau > 0 the largest
  // weight of a row is 2^delta instead of exactly 1. FP8 takes tau = 0.75
  // (P * 256 * 2^0.75 <= 431 stays below e4m3's 448); bf16 keeps tau = 0, as
  // the bf16 rounding of a dominant weight would eat most of the 1e-2 margin
  // of causal rows with a handful of keys.
  constexpr float kTau = 0.25f * TAUQ;
  static_assert(TAUQ == 0 || (DT == kFP8 && TAUQ <= 3), "tau > 0: FP8 only, P * 256 * 2^tau below 448");
  // a negative scale is folded into Q (sign flip, exact), so c > 0 below
  const bool neg_scale = c < 0.0f;
  c = fabsf(c);
  if (c == 0.0f) c = 1e-30f;

  Op qop[QK_STEPS];
  // MX: lane half hh holds 16-byte chunks 4kk + 2x + hh of the row (the scaled
  // MFMA's contraction order, so each hardware block is 32 consecutive head
  // dims); otherwise chunks 4kk + 2hh + x (bf16: 2kk + hh). A and B use the
  // same order, which is all the unscaled product needs.
  int q_sc = 0;
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qg, head_bytes);
    const uint32_t qoff = (uint32_t)my_q * ROW + (MX ? 16 : KPL * ES) * hh;
#pragma unroll
    for (int kk = 0; kk < QK_STEPS; ++kk)
#pragma unroll
      for (int x = 0; x < Op::DW / 4; ++x) {
        const uint32_t xo = MX ? 32 * x : 16 * x;
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + kk * 2 * KPL * ES + xo, 0, 0);
#pragma unroll
        for (int y = 0; y < 4; ++y) qop[kk].w[4 * x + y] = w[y];
      }
    if constexpr (MX) {
      // the row's D/32 scale bytes; byte 2kk of q_sc is the block of step kk
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(p.q_scale + (size_t)bh * N * (D / 32), (uint32_t)N * (D / 32));
      q_sc = (int)(__builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)my_q * (D / 32), 0, 0) >> (8 * hh));
    }
    if (neg_scale) {
      constexpr uint32_t sign = ES == 2 ? 0x80008000u : 0x80808080u;
#pragma unroll
      for (int kk = 0; kk < QK_STEPS; ++kk)
#pragma unroll
        for (int w = 0; w < Op::DW; ++w) qop[kk].w[w] ^= sign;
    }
  }

  int T = (N + BN - 1) / BN;
  if constexpr (CAUSAL) {
    const int last = (q0 + BM - 1) / BN + 1;
    T = T < last ? T : last;
  }
  int j_begin, j_end;
  key_tile_range<SPLIT, BN>(p, sp, T, j_begin, j_end);

  // ---- DMA: instruction t of this wave fills LDS chunks 64 (wave + NWAVES t) + lane ----
  // row r = chunk / CPR, physical column chunk pc -> logical pc ^ f(r); rows of
  // instruction t are those of t = 0 plus 64 NWAVES t / CPR (a multiple of 8, so
  // f is unchanged): instruction t reads at the lane offsets of t = 0 plus
  // t T_ROWS ROW bytes, under one descriptor per tile.
  const int dma_row = (64 * wave + lane) / CPR;
  const int dma_pc = lane % CPR;
  const uint32_t k_goff = (uint32_t)dma_row * ROW + 16 * (dma_pc ^ swz_k<DT, D>(dma_row));
  const uint32_t v_goff = (uint32_t)dma_row * ROW + 16 * (dma_pc ^ swz_v<DT, D>(dma_row));
  constexpr int T_ROWS = 64 * NWAVES / CPR;      // rows between instruction t and t+1
  static_assert(T_ROWS % 16 == 0, "swizzle period");

  // one descriptor per tile for K and one for V (base at the tile's first
  // row, range up to the end of the head: rows >= N read as zero); the
  // tile's instructions t differ only in their lane offsets t T_ROWS ROW
  uint32_t k_goff_t[NINSTR], v_goff_t[NINSTR];
#pragma unroll
  for (int t = 0; t < NINSTR; ++t) {
    k_goff_t[t] = k_goff + (uint32_t)(t * T_ROWS * ROW);
    v_goff_t[t] = v_goff + (uint32_t)(t * T_ROWS * ROW);
  }
  auto issue_tile = [&](int jt, int buf) {
    const int kbase = jt * BN;
    unsigned char* st = smem + buf * STAGE;
    const uint32_t bytes = (uint32_t)(N - kbase) * ROW;     // kbase < N for every tile issued
    const i32x4_t rk = dma_rsrc(Kg + (size_t)kbase * ROW, bytes);
    const i32x4_t rv = dma_rsrc(Vg + (size_t)kbase * ROW, bytes);
#pragma unroll
    for (int t = 0; t < NINSTR; ++t) {
      const uint32_t lds = (uint32_t)(uintptr_t)(lds_void_ptr)(st + 1024 * (wave + NWAVES * t));
      // the first use of each descriptor waits out a VALU write of its SGPRs
      if (t == 0) {
        lds_dma16_rsrc<4>(rk, lds, k_goff_t[0]);
        lds_dma16_rsrc<4>(rv, lds + TILE, v_goff_t[0]);
      } else {
        lds_dma16_rsrc<0>(rk, lds, k_goff_t[t]);
        lds_dma16_rsrc<0>(rv, lds + TILE, v_goff_t[t]);
      }
    }
    if constexpr (MX) {
      if (wave == 0) {
        const uint32_t lds = (uint32_t)(uintptr_t)(lds_void_ptr)(st + 2 * TILE);
        const int kb0 = kbase / 32, nkb = (N + 31) / 32;
        lds_dma4(p.k_scale + ((size_t)bkv * N + kbase) * (D / 32), (uint32_t)(N - kbase) * (D / 32), lds,
                 4 * lane);
        lds_dma4(p.v_scale + ((size_t)bkv * nkb + kb0) * D, (uint32_t)(nkb - kb0) * D, lds + SC_K, 4 * lane);
      }
    }
  };

  // ---- MFMA operand read bases ----
  // K: row r = 32b + l32 (same swizzle as row l32); bf16 chunk 2kk + h, fp8
  // chunks 4kk + 2h + x
  const int gk = swz_k<DT, D>(l32);
  constexpr int NKB = DT == kFP8 ? 2 * QK_STEPS : (QK_STEPS < 4 ? QK_STEPS : 4);
  uint32_t kb[NKB];
#pragma unroll
  for (int u = 0; u < NKB; ++u) {
    const int lc = DT == kFP8 ? (MX ? 4 * (u >> 1) + 2 * (u & 1) + hh : 4 * (u >> 1) + 2 * hh + (u & 1))
                              : (2 * u + hh);
    kb[u] = (uint32_t)l32 * ROW + 16 * (lc ^ gk);
    // one register per base: left visible, the compiler splits it into a row
    // part and a chunk part and spends two VALU ops per base and tile
    asm volatile("" : "+v"(kb[u]));
  }
  // V (transpose reads): group g = lane / 16, j = lane % 16
  const int vg = lane >> 4, vj = lane & 15, va = vg & 1;
  uint32_t vb[4];
  if constexpr (DT == kBF16) {
    // source row 4h + e (+ 16n + 8t), e = j/4; columns 32mb + 16a + 4q, q = j%4
    const int e = vj >> 2, q = vj & 3, r0 = 4 * hh + e;
    const int x = 2 * va + (q >> 1);
#pragma unroll
    for (int m1 = 0; m1 < 2; ++m1)
      vb[m1] = TILE + (uint32_t)r0 * ROW + 16 * ((4 * m1 + x) ^ swz_v<DT, D>(r0)) + 8 * (q & 1);
  } else {
    // source row 4h + e%4 + 8(e/4) (+ 16t), e = j/2; columns 32mb + 16a + 8q, q = j%2
    const int e = vj >> 1, q = vj & 1, r0 = 4 * hh + (e & 3) + 8 * (e >> 2);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      vb[mb] = TILE + (uint32_t)r0 * ROW + 16 * ((2 * mb + va) ^ swz_v<DT, D>(r0)) + 8 * q;
  }

  f32x16 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[mb][r] = 0.0f;
  // Reference max m_ref (log2 units) that p, l and O are taken against,
  // m_sub = m_ref - bias, and thr = the raw score above which a row's tile max
  // moves the reference: tau above it (-inf until the row has one).
  float m_ref = -__builtin_inff();
  float m_sub = 0.0f;
  float thr = -__builtin_inff();
  float l_run = 0.0f;
  const float inv_c = 1.0f / c;
  constexpr float masked_raw = -__builtin_inff();
  constexpr int kReadsPerOp = Op::DW / 4;

  // every wave issues 2 NINSTR DMA loads per tile. The prologue waits for all
  // of its loads (Q included): the compiler's own vmcnt bookkeeping, blind to
  // the DMAs, then has nothing pending inside the loop.
  if (j_begin < j_end) issue_tile(j_begin, 0);
  if constexpr (NSTAGE == 3) {
    if (j_begin + 1 < j_end) issue_tile(j_begin + 1, 1);
  }
  wait_vmcnt<0>();
  __syncthreads();

  int buf = 0;   // stage of tile j
  for (int j = j_begin; j < j_end; ++j) {
    const int ahead = j + NSTAGE - 1;
    auto issue_ahead = [&]() {
      if (ahead < j_end) {
        int nb = buf + NSTAGE - 1;
        nb = nb >= NSTAGE ? nb - NSTAGE : nb;
        issue_tile(ahead, nb);
      }
    };
    if constexpr (!LATE_DMA) issue_ahead();
    const int kbase = j * BN;
    const bool wave_active = !CAUSAL || kbase <= q0w + 31;
    const unsigned char* st = smem + buf * STAGE;
    f32x16 s[NB];
    if (wave_active) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[b][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < QK_STEPS; ++kk)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          Op a;
#pragma unroll
          for (int x = 0; x < kReadsPerOp; ++x) {
            const int u = DT == kFP8 ? 2 * kk + x : (kk & 3);
            const int imm = DT == kFP8 ? 0 : 128 * (kk >> 2);
            const u32x4 w = *(const u32x4*)(st + kb[u] + imm + b * 32 * ROW);
#pragma unroll
            for (int y = 0; y < 4; ++y) a.w[4 * x + y] = w[y];
          }
          if constexpr (MX) {
            // the key row's D/32 scale bytes, block hh of step kk at byte 2kk
            const int k_sc = (int)(*(const uint32_t*)(st + 2 * TILE + 4 * (32 * b + l32)) >> (8 * hh));
            if (kk == 0)
              mfma_fp8_scaled<0, 0>(a, qop[kk], s[b], k_sc, q_sc);
            else
              mfma_fp8_scaled<2, 2>(a, qop[kk], s[b], k_sc, q_sc);
          } else {
            mfma<DT>(a, qop[kk], s[b]);
          }
        }
      if constexpr (LOOK > 0) interleave_reads_with_mfma<QK_STEPS * NB, kReadsPerOp, LOOK>();
    }
    if constexpr (LATE_DMA) issue_ahead();
    if (wave_active) {
      const bool need_mask = (kbase + BN > N) || (CAUSAL && kbase + BN - 1 > q0w);
      // the mask and the rescale below are rare: marked unlikely, their code
      // goes out of line and the common path runs without a taken branch
      // (+0.5% on the 56 x 30272 shape, bf16 and FP8)
      if (__builtin_expect(need_mask, 0)) {
        asm volatile("" ::: "memory");
        int lim = N - kbase - 4 * hh;
        if constexpr (CAUSAL) {
          const int lim_c = my_q - kbase - 4 * hh + 1;
          lim = lim < lim_c ? lim : lim_c;
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rel = 32 * b + 8 * (r >> 2) + (r & 3);
            s[b][r] = rel < lim ? s[b][r] : masked_raw;
          }
      }
      // the lane's max of its raw scores; a tile where no row's max exceeds
      // the reference by more than tau takes p against the reference as it
      // stands. Both halves of a row hold its threshold, so the test needs no
      // exchange: the row max (the two halves combined) is formed only when
      // the reference moves.
      const float lane_ext = max_reduce<NB * 16>([&](int i) { return s[i >> 4][i & 15]; });
      if (__builtin_expect(__any(lane_ext > thr), 0)) {
        // a new exact reference for every row of the wave, O rescaled to it
        const float ext = swap_halves_max(lane_ext);
        const float m_new = vmax(m_ref, ext * c);
        // a causal chunk can start above a row's diagonal: until the row meets
        // a valid key its reference stays -inf, and a zero subtrahend keeps
        // p = 0 and alpha = 0
        const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_use);
        m_ref = m_new;
        m_sub = m_use - kPBias;
        thr = m_new == -__builtin_inff() ? -__builtin_inff() : (m_use + kTau) * inv_c;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
        l_run *= alpha;
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[b][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], c, -m_sub));
      float ps[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
      for (int i = 4; i < NB * 16; ++i) ps[i & 3] += s[i >> 4][i & 15];
      l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      Op pop[PV_STEPS];
#pragma unroll
      for (int n = 0; n < PV_STEPS; ++n) {
        if constexpr (DT == kBF16) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int r0 = n * KPL + 2 * w;
            pop[n].w[w] = pack_bf16(s[r0 >> 4][r0 & 15], s[(r0 + 1) >> 4][(r0 + 1) & 15]);
          }
        } else {
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const int r0 = n * KPL + 4 * w;
            // both halves are overwritten below: an opaque, unset word spares the
            // v_mov that clearing it would cost
            int v;
            asm volatile("" : "=v"(v));
            v = __builtin_amdgcn_cvt_pk_fp8_f32(s[r0 >> 4][r0 & 15], s[(r0 + 1) >> 4][(r0 + 1) & 15], v, false);
            v = __builtin_amdgcn_cvt_pk_fp8_f32(s[(r0 + 2) >> 4][(r0 + 2) & 15], s[(r0 + 3) >> 4][(r0 + 3) & 15], v, true);
            pop[n].w[w] = (uint32_t)v;
          }
        }
      }
      // O^T += V^T P^T with transpose reads
#pragma unroll
      for (int n = 0; n < PV_STEPS; ++n)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          Op a;
          if constexpr (DT == kBF16) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const unsigned char* src = st + vb[mb & 1] + 128 * (mb >> 1) + (16 * n + 8 * t) * ROW;
              const s16x4_t v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)src);
              const i32x2_t v2 = __builtin_bit_cast(i32x2_t, v4);
              a.w[2 * t] = (uint32_t)v2[0];
              a.w[2 * t + 1] = (uint32_t)v2[1];
            }
          } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const unsigned char* src = st + vb[mb] + (64 * n + 16 * t) * ROW;
              const i32x2_t v2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_ptr)src);
              a.w[2 * t] = (uint32_t)v2[0];
              a.w[2 * t + 1] = (uint32_t)v2[1];
            }
          }
          if constexpr (MX) {
            // keys 64n + 32hh .. + 31 of the tile form block hh of this step;
            // the scale of head dim 32mb + l32 in that key block; P unscaled
            const int v_sc = st[2 * TILE + SC_K + (2 * n + hh) * D + 32 * mb + l32];
            mfma_fp8_scaled<0, 0>(a, pop[n], oacc[mb], v_sc, 0x7F7F7F7F);
          } else {
            mfma<DT>(a, pop[n], oacc[mb]);
          }
        }
    }
    // tile j+1 must have landed; with three stages tile j+2 may stay in flight
    if constexpr (NSTAGE == 3) {
      if (j + 2 < j_end)
        wait_vmcnt<2 * NINSTR>();
      else
        wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    buf = buf + 1 == NSTAGE ? 0 : buf + 1;
  }

  const float l_tot = swap_halves_sum(l_run);
  if constexpr (SPLIT) {
    store_partial<MB>(p, sp, bh, my_q, hh, oacc, l_tot, m_ref - kPBias, dv);
    return;
  }
  const float inv = dv / l_tot;
  if (my_q < N) {
    if (hh == 0)
      p.lse[(size_t)bh * N + my_q] = (m_ref - kPBias + __builtin_amdgcn_logf(l_tot)) * 0.6931471805599453f;
    const size_t obase = ((size_t)bh * N + my_q) * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * mb + 8 * jj + 4 * hh;
        uint2 pk;
        pk.x = pack_bf16(oacc[mb][4 * jj + 0] * inv, oacc[mb][4 * jj + 1] * inv);
        pk.y = pack_bf16(oacc[mb][4 * jj + 2] * inv, oacc[mb][4 * jj + 3] * inv);
        *(uint2*)((unsigned short*)p.o + obase + d0) = pk;
      }
  }
}

}  // namespace fa
