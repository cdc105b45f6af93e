// Stage 2: block-sparse causal prefill attention with the fused mean correction.
//
// Method: "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context LLM
// Serving" (metallab.ai paper digest):
//   Figure 3  Stage 2 computes exact attention over the CSR-selected blocks
//             while unselected blocks are compensated by the mean-correction
//             path; both streams merge inside one online softmax.
//   Figure 4  a pruned block J contributes |B_J| exp(s_J) (v_bar_J, 1): here
//             the logit sm * q_i . k_bar_J + ln n_J on value v_bar_J.
//   Figure 1 and "What they did"  PackGQA: the G query heads of one KV head
//             are packed into one tile so each K/V tile is fetched once for
//             them.
//
// gfx950 design (not a translation of the pages' Hopper kernel):
//   * One workgroup = 8 waves (two per SIMD) = 256 packed query rows of one
//     (KV head h, query block I): wave w owns 32 consecutive tokens of one
//     query head. G*B rows per (h, I) are split over ceil(G*B/256) workgroups.
//   * Transposed products keep every lane on one query: S^T = K Q^T and
//     O^T = V^T P^T with v_mfma_f32_32x32x16_bf16 (QK^T of FP8 inputs with
//     v_mfma_f32_32x32x64_f8f6f4, below). A lane (column c, half hf)
//     holds the scores and output dims of query c, so row max and row sum are
//     in-lane plus one v_permlane32_swap, and the probabilities feed the PV
//     product straight from registers (the PV contraction index is relabelled
//     to match the score accumulator layout).
//   * Work items: the CSR row's key blocks, then correction chunks of 64
//     pooled columns: the row's pruned blocks in column order, gathered by
//     DMA from a list the waves build in LDS from a bitmap of the row, each
//     with bias log2(n_J) (-inf for unused columns of the last chunk). The kept blocks
//     between the row's first and last item run through a pipelined
//     instantiation without score adjustments; the diagonal block, the last
//     kept block and the correction chunks through a general one.
//   * Staging is direct HBM -> LDS (buffer_load ... lds / global_load_lds,
//     16 bytes per lane) into double-buffered tiles, so no registers carry
//     K or V. A tile stores rows in groups of four: group g (rows 4g..4g+3)
//     occupies 1088 bytes, chunk-major (16-byte chunk c of row 4g+i at
//     64c + 16i) with 64 bytes of padding, which is exactly the order one
//     wave's 1 KiB DMA writes when lane l fetches chunk l/4 of row 4g + l%4.
//     K operand reads (16 bytes: row, chunk 2ks+hf) are then base + 128 ks
//     immediates, and V^T operands come from the gfx950 transposing read
//     ds_read_b64_tr_b16 (lane j of a 16-lane group reads 4 dims of one key;
//     the hardware hands lane i dim i of 4 consecutive keys), also at
//     immediate offsets; both are bank-conflict free.
//   * Pooled items read bf16 copies of k_bar, v_bar (scaled to code units for
//     FP8) that a small conversion kernel writes into the workspace.
//   * FP8 (E4M3) inputs: QK^T of the kept blocks runs on the codes with
//     v_mfma_f32_32x32x64_f8f6f4 (products of two codes are exact in fp32, so
//     the scores are those of the widened codes, at twice the bf16 rate); K
//     tiles hold the FP8 rows (half the DMA and LDS bytes). P V stays bf16:
//     P rounded to E4M3 (3 mantissa bits) moves the output about 20 times
//     as far as bf16 P does (max-abs 0.027 against 0.0015 on unit-variance
//     V, 4K keys). V is widened once by the conversion kernel (exactly),
//     and correction chunks multiply the bf16 pooled rows by Q widened in
//     registers.
//   * Online softmax in base 2, updated per 64-key half of an item: one fma +
//     exp2 per score against the running max as it stands, fp32 row sums. A
//     half takes its own max only when a probability exceeds 2^64 (the row's
//     first keys, or scores that grew by more than 64 in log2 units); the
//     running max then moves if the half's max exceeds it by more than 8, and
//     the output is rescaled. Probabilities stay below 2^64 and row sums far
//     inside fp32; the result is exact after the final division.
//   * Workgroups run heaviest first (query block index descending over the
//     ragged batch). Consecutive ids cycle over KV heads, and the head of each
//     id slot rotates every kRotateSpan / Hkv query blocks: the round-robin XCD
//     dispatch then keeps a head's K/V in one L2 across neighbouring rows
//     while every XCD sees every head (the heads' kept counts differ by up
//     to 14 % at 128K, and a fixed head per XCD let the busiest one set the
//     kernel time: 9.62 -> 8.61 ms). The period is 1024 / Hkv query blocks
//     (128 with 8 KV heads): the kernel time is level with shorter periods
//     (8.95 against 8.94 ms for 16 and 8.86 for 64 at 128K, interleaved), and
//     a head stays on an XCD long enough for its kept tiles to be reused from
//     L2 (L2 misses 7.11 -> 5.44 GB per launch against a period of 16).
//   * Split-KV ([digest] Table 7: count-balanced CSR splits): when a launch
//     has too few rows to fill the chip, each row's item list is cut into
//     `splits` consecutive parts of equal cost (an exact block counts 2, a
//     64-column correction chunk 1), one workgroup per part. A part writes its
//     normalised fp32 output and its log2-sum-exp to the workspace, and
//     merge_kernel combines the parts by their log-sum-exp.
#include "common.h"
#include "launch.h"

namespace fpv2 {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWG = kWaves * 32;
constexpr int kSlab = 4 * kWaves;       // tile rows one DMA instruction of every wave fills
constexpr int kPC = 64;                 // pooled columns per correction item
constexpr int kQuad = 4 * 256 + 64;     // LDS bytes of a group of four 256-byte rows
// K / V layouts (the PAGED template argument): contiguous, paged with any
// page size (a page-table lookup per row), paged with a page size that is a
// multiple of 4 (one lookup per four rows, which lets the DMA be spread).
constexpr int kContig = 0, kPagedAny = 1, kPaged4 = 2;
// FP8 K tiles hold the codes themselves (128-byte rows) in groups of eight
// rows: 1024 bytes chunk-major (16-byte chunk c of row 8g + i at 128c + 16i),
// the order one wave's 1 KiB DMA writes when lane l fetches chunk l/8 of row
// 8g + l%8, plus 128 bytes of padding, so the sixteen lanes of one operand
// read (rows c .. c+15, one chunk) hit distinct banks.
constexpr int kOct = 8 * 128 + 128;
constexpr int kSlab8 = 8 * kWaves;      // FP8 K rows one DMA instruction of every wave fills

// A work-unit slot keeps its KV head for kRotateSpan / Hkv query blocks (see
// decode_work).
constexpr int kRotateSpan = 1024;
constexpr int kColCache = 1024;         // CSR columns cached in LDS
constexpr int kPList = 2048;            // pruned blocks listed in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;
constexpr float kSlack = 8.0f;          // lazy-rescale threshold of the running max (log2)

// Eight probabilities as one bf16 P operand, added in fp32 to the row sum.
// (Summing the rounded bf16 values instead, two per v_dot2_f32_bf16, saves
// 16 VALU instructions per half but moves the log-sum-exp by up to 2^-9
// relative, outside a 1e-3 bound for rows with few keys.)
__device__ __forceinline__ bf16x8 pack_probs(const float (&pv)[8], float& lsum) {
#pragma unroll
  for (int t = 0; t < 8; ++t) lsum += pv[t];
  const bf16x4 lo = __builtin_convertvector(f32x4{pv[0], pv[1], pv[2], pv[3]}, bf16x4);
  const bf16x4 hi = __builtin_convertvector(f32x4{pv[4], pv[5], pv[6], pv[7]}, bf16x4);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) void* gbl_ptr;

template <int BLK>
struct Tile {
  static constexpr int kBytes = BLK / 4 * kQuad;
  static constexpr int kWords = kBytes / 16;
  static_assert(BLK / 8 * kOct <= kBytes, "FP8 K tile");
};

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Buffer resource for raw 16-byte loads: base, byte range [0, num_records).
// Lanes whose offset lies past the range read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, int num_records) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_records, 0x00020000);
}

// Per-workgroup constants of the row being processed (all wave-uniform).
struct RowCtx {
  int r, I, h, L;
  int n_exact;          // CSR entries (key blocks) of the row
  int n_corr;           // pruned causal blocks: one correction column each
  bool listed;          // the pruned blocks are listed in LDS (n_corr <= kPList)
  int n_items;          // plus the correction chunks
  const int32_t* cols;  // CSR row (nullptr in dense mode)
  int64_t pooled_row0;  // row h * kpitch + prow_off[r] of k_bar / v_bar
  int64_t tok_base;     // first key token of the request (contiguous K / V)
};

// Combine lane c with lane c+32 (the two key halves of one query) with the
// gfx950 cross-half swap: with both operands x, the two results hold
// x[0..31] and x[32..63] on every lane.
__device__ __forceinline__ float max_halves(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// Per-wave online-softmax state for 32 query rows.
template <int BLK>
struct WaveState {
  bf16x8 qf[kHeadDim / 16];  // B operand of S^T = K Q^T, one per 16-dim step (bf16)
  i32x8 q8[kHeadDim / 64];   // FP8: the codes as B operand, one per 64-dim step
  f32x16 o[kHeadDim / 32];   // O^T accumulators, one per 32-dim tile
  float m;                   // running max (log2 units)
  float l;                   // this lane's partial row sum
};

// Probabilities 2^(s sc - m) of one 64-key half as bf16 P operands; returns
// this lane's fp32 sum of them.
__device__ __forceinline__ float half_probs(const f32x16 (&s)[2], float sc, float neg_m, bf16x8 (&pf)[2][2]) {
  float lsum = 0.f;
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      float pv[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) pv[t] = __builtin_amdgcn_exp2f(fmaf(s[t2][8 * s2 + t], sc, neg_m));
      pf[t2][s2] = pack_probs(pv, lsum);
    }
  }
  return lsum;
}

// Online-softmax update of one half of scores s (s sc in log2 units). The
// probabilities are taken against the running max m as it stands; only when
// one of them exceeds 2^64 (always on the row's first keys, where m is unset)
// does the half take its max, move m if that max exceeds it by more than
// kSlack, rescale O and l, and take them again. So m may trail the true
// maximum by up to 64: every probability stays below 2^64 and every row sum
// below 2^86, far inside fp32, and the result is the same softmax after the
// final division. The common path spends no instruction on the maximum.
template <int BLK>
__device__ __forceinline__ void softmax_half(WaveState<BLK>& ws, const f32x16 (&s)[2], float sc, bf16x8 (&pf)[2][2]) {
  constexpr float kPMax = 18446744073709551616.0f;  // 2^64
  float lsum = half_probs(s, sc, -ws.m, pf);
  if (__ballot(!(lsum <= kPMax)) != 0) {
    float mx = kNegBig;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[t2][e]);
    mx = max_halves(mx * sc);
    const float m_new = mx > ws.m + kSlack ? mx : ws.m;
    if (__ballot(m_new != ws.m) != 0) {
      const float corr = __builtin_amdgcn_exp2f(ws.m - m_new);
      ws.l *= corr;
#pragma unroll
      for (int dt = 0; dt < kHeadDim / 32; ++dt) ws.o[dt] *= corr;
    }
    ws.m = m_new;
    lsum = half_probs(s, sc, -m_new, pf);
  }
  ws.l += lsum;
}

// Item kinds: a selected key block off the diagonal (all keys visible), the
// diagonal block (causal mask from tile kt_lim on), or a chunk of pooled
// columns (logit s*sl2 + bias[col]; columns past the chunk end have bias
// -inf).
enum ItemKind { kExact = 0, kDiag = 1, kPooled = 2, kDiagFirst = 3 };  // kDiagFirst: the diagonal of a
                                                                    // request's first query block

// V^T operand for PV job j of a half (tile 2hh + (j >> 3), MFMA s2 = (j >> 2) & 1,
// dims 32 (j & 3) ..): keys 16 s2 + 4 hf + 0..3 and + 8..11 of the tile, each
// four keys one transposing read.
__device__ __forceinline__ bf16x8 v_operand(const uint8_t* vh, int j) {
  const uint8_t* a = vh + (j >> 3) * 8 * kQuad + ((j >> 2) & 1) * 4 * kQuad + (j & 3) * 256;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)a);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(a + 2 * kQuad));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// PV of a half: job j = (tile t2 = j >> 3, s2 = (j >> 2) & 1, dt = j & 3); the
// four output accumulators rotate, so consecutive MFMAs are independent, and
// V operands are read DEPTH jobs ahead (the first DEPTH are already in vf).
template <int NJ, int DEPTH>
__device__ __forceinline__ void pv_jobs(f32x16 (&o)[kHeadDim / 32], bf16x8 (&vf)[DEPTH], const bf16x8 (&pf)[2][2],
                                        const uint8_t* vh) {
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    o[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j % DEPTH], pf[j >> 3][(j >> 2) & 1], o[j & 3], 0, 0, 0);
    if (j + DEPTH < NJ) vf[j % DEPTH] = v_operand(vh, j + DEPTH);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// bf16 K operand of QK job j of a half (tile 2hh + (j & 1), 16-dim step
// ks = j >> 1): 16 bytes of row c. The lane's dims of step ks are those its
// Q operand holds: 16 ks + 8 hf .. (chunk 2 ks + hf) for bf16 Q; for FP8 Q,
// whose codes are held per 64-dim step, 64 (ks / 4) + 32 hf + 8 (ks % 4) ..
// (chunk 8 (ks / 4) + 4 hf + ks % 4); the lane's hf part is in its base.
template <bool F8>
__device__ __forceinline__ bf16x8 k_operand(const uint8_t* kh, int j) {
  const int ks = j >> 1;
  const int off = F8 ? 512 * (ks >> 2) + 64 * (ks & 3) : 128 * ks;
  return *reinterpret_cast<const bf16x8*>(kh + (j & 1) * 8 * kQuad + off);
}

// QK^T of one half: two accumulation chains, K operands read kDepth ahead.
template <int DEPTH, bool F8>
__device__ __forceinline__ void qk_half(const bf16x8 (&qf)[kHeadDim / 16], const uint8_t* kh, f32x16 (&s)[2]) {
  constexpr int NJ = 2 * (kHeadDim / 16);
  bf16x8 kf[DEPTH];
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) kf[j] = k_operand<F8>(kh, j);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    s[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j % DEPTH], qf[j >> 1], j < 2 ? f32x16{} : s[j & 1], 0, 0, 0);
    if (j + DEPTH < NJ) kf[j % DEPTH] = k_operand<F8>(kh, j + DEPTH);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// FP8 K operand of QK job j of a half (tile 2hh + (j & 1), dims 64 (j >> 1)
// + 32 hf .. + 31): 32 bytes of row c, chunks 4 (j >> 1) + 2 hf and the next.
__device__ __forceinline__ i32x8 k8_operand(const uint8_t* kh, int j) {
  const uint8_t* a = kh + (j & 1) * 4 * kOct + (j >> 1) * 512;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(a);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(a + 128);
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// bf16 K operand of QK job j of a half, read from an FP8 K tile and widened
// exactly: the 8 codes of row c at the dims widen_q gives the lane's Q
// operand of step ks = j >> 1, 64 (ks / 4) + 32 hf + 8 (ks % 4) .. + 7, lie
// in one 16-byte chunk of the row (the lane's hf part is in its base).
__device__ __forceinline__ bf16x8 k8w_operand(const uint8_t* kh, int j) {
  const int ks = j >> 1;
  const uint2 w = *reinterpret_cast<const uint2*>(kh + (j & 1) * 4 * kOct + (4 * (ks >> 2) + ((ks & 3) >> 1)) * 128 +
                                                  8 * (ks & 1));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// QK^T of one half from an FP8 K tile on the bf16 matrix cores (Q and K
// widened exactly): the sums are those of fp32 arithmetic, where the FP8
// matrix cores keep about 12 bits below each 64-term step's largest product
// (an in-bounds probe measured errors up to 2^-12.1 of it, 15 code units on
// a sum of 1e5, against 0.02 for the bf16 products of the same codes).
template <int DEPTH>
__device__ __forceinline__ void qk_half8w(const bf16x8 (&qw)[kHeadDim / 16], const uint8_t* kh, f32x16 (&s)[2]) {
  constexpr int NJ = 2 * (kHeadDim / 16);
  bf16x8 kf[DEPTH];
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) kf[j] = k8w_operand(kh, j);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    s[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j % DEPTH], qw[j >> 1], j < 2 ? f32x16{} : s[j & 1], 0, 0, 0);
    if (j + DEPTH < NJ) kf[j % DEPTH] = k8w_operand(kh, j + DEPTH);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// S^T += K Q^T over 64 dims on E4M3 codes (v_mfma_f32_32x32x64_f8f6f4, both
// operands FP8, no block scales). The products of two codes are exact, but
// the instruction sums them with about 12 bits below the largest (see
// qk_half8w), which the kept blocks off the diagonal accept for the FP8 rate.
__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The FP8 Q codes widened to bf16 (exactly: every E4M3 value is a bf16
// value) as B operands of bf16 products, 8 codes per 16-dim step in the
// order k_operand<true> reads the K side.
__device__ __forceinline__ void widen_q(const i32x8 (&q8)[kHeadDim / 64], bf16x8 (&qf)[kHeadDim / 16]) {
#pragma unroll
  for (int ks = 0; ks < kHeadDim / 16; ++ks) {
    const uint32_t lo = (uint32_t)q8[ks >> 2][2 * (ks & 3)], hi = (uint32_t)q8[ks >> 2][2 * (ks & 3) + 1];
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    qf[ks] = bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
}

// FP8 QK^T of one half: tiles 2hh, 2hh+1 in two 64-dim steps each (four
// MFMAs, two chains); the second step's operands load under the first.
__device__ __forceinline__ void qk_half8(const i32x8 (&q8)[kHeadDim / 64], const uint8_t* kh, f32x16 (&s)[2]) {
  i32x8 kf[2] = {k8_operand(kh, 0), k8_operand(kh, 1)};
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    s[j & 1] = mfma_f8(kf[j & 1], q8[j >> 1], j < 2 ? f32x16{} : s[j & 1]);
    if (j < 2) kf[j & 1] = k8_operand(kh, j + 2);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One item for one wave, processed in 64-key halves (each: QK^T of two
// 32-key tiles, online-softmax update, PV), which keeps 32 score registers
// live instead of 64. Every half computes both of its tiles: on the diagonal
// the causal mask also covers a tile past the query block's last visible key,
// and a pooled chunk is one half whose unused columns have bias -inf (their
// staged rows are zeros), so the code has no data-dependent tile skips, and
// the three item kinds share one copy of the MFMA code (their differences are
// short wave-uniform branches on the scores).
// kt_lim (diagonal only): the tile that holds the query's own position.
// Operand reads run a few MFMAs ahead of their use; the schedule is pinned
// with scheduling fences because the compiler otherwise places every LDS read
// right before its MFMA and exposes the LDS latency each time.
// F8: kept blocks are FP8 K tiles (operand base lk8), correction chunks bf16
// tiles of the pooled rows (base lk).
template <int BLK, bool EXACT, bool F8>
__device__ __forceinline__ void attend_item(WaveState<BLK>& ws, const uint8_t* kb, const uint8_t* vt,
                                            const float* bias, int kind, int kt_lim, int tq, float sl2, int lk,
                                            int lk8, int lv, int hf) {
  constexpr int kDepth = 4;  // operand reads in flight
  if (EXACT) kind = kExact;
  const bool first = kind == kDiagFirst;
  if (first) kind = kDiag;
  const int nh = kind == kPooled ? 1 : BLK / 64;
  // Pooled scores are turned into log2-unit logits with their bias before
  // the max; exact scores are scaled after it.
  const float sc = kind == kPooled ? 1.0f : sl2;
#pragma unroll
  for (int hh = 0; hh < BLK / 64; ++hh) {
    if (hh >= nh || (kind == kDiag && 2 * hh > kt_lim)) break;
    // QK^T of tiles 2hh, 2hh+1 (rows 32kt + c of a tile).
    f32x16 s[2];
    if constexpr (F8) {
      if (kind != kPooled && !first) {
        qk_half8(ws.q8, kb + lk8 + (2 * hh) * 4 * kOct, s);
      } else if (first) {
        // The diagonal of a request's first query block on the bf16 matrix
        // cores: those queries see no other keys, so their log-sum-exp is
        // this block's scores alone and can lie near 0, where a relative
        // bound needs the scores to fp32 accuracy. Later rows sum over at
        // least one more block.
        bf16x8 qw[kHeadDim / 16];
        widen_q(ws.q8, qw);
        qk_half8w<kDepth>(qw, kb + lk8 + (2 * hh) * 4 * kOct, s);
      } else {
        // The pooled rows are bf16: Q widened for this chunk (not kept, to
        // leave the registers to the kept blocks' pipeline).
        bf16x8 qw[kHeadDim / 16];
        widen_q(ws.q8, qw);
        qk_half<kDepth, true>(qw, kb + lk + (2 * hh) * 8 * kQuad, s);
      }
    } else {
      qk_half<kDepth, false>(ws.qf, kb + lk + (2 * hh) * 8 * kQuad, s);
    }
    // The first V operands load while the softmax runs.
    const uint8_t* vh = vt + lv + (2 * hh) * 8 * kQuad;
    bf16x8 vf[kDepth];
#pragma unroll
    for (int j = 0; j < kDepth; ++j) vf[j] = v_operand(vh, j);
    __builtin_amdgcn_sched_barrier(0);
    if (kind == kPooled) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 bb = *reinterpret_cast<const float4*>(&bias[t2 * 32 + i * 8 + hf * 4]);
          s[t2][4 * i + 0] = fmaf(s[t2][4 * i + 0], sl2, bb.x);
          s[t2][4 * i + 1] = fmaf(s[t2][4 * i + 1], sl2, bb.y);
          s[t2][4 * i + 2] = fmaf(s[t2][4 * i + 2], sl2, bb.z);
          s[t2][4 * i + 3] = fmaf(s[t2][4 * i + 3], sl2, bb.w);
        }
      }
    } else if (kind == kDiag && 2 * hh + 1 >= kt_lim) {
      // Keys past the query; only the half holding tile kt_lim has any.
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if ((2 * hh + t2) * 32 + i * 8 + hf * 4 + jj > tq) s[t2][4 * i + jj] = -INFINITY;
    }
    bf16x8 pf[2][2];
    softmax_half(ws, s, sc, pf);
    __builtin_amdgcn_sched_barrier(0);
    pv_jobs<16, kDepth>(ws.o, vf, pf, vh);
  }
}

// Several requests: (query block I, request r) of unit row pk. With C(x) the
// number of (request q, query block I' of q) with I' > x, non-increasing in
// x, I is the smallest x with C(x) <= pk, and r the (pk - C(I))-th request
// (in order) that has query block I. Lane q (and q + 64) holds request q's
// key-block count and first query block; each round of the search lets the 64
// lanes evaluate C at 64 evenly spaced candidates (the request values
// broadcast by readlane), so three rounds cover 2^18 blocks, with no chain of
// dependent memory loads.
__device__ __forceinline__ void decode_multi(const ReqTable& rt, int pk, int& I, int& r) {
  const int lane = threadIdx.x & 63;
  const int R = rt.R;
  int nbA = 0, q0A = 0, nbB = 0, q0B = 0;
  if (lane < R) {
    nbA = rt.kblk_off[lane + 1] - rt.kblk_off[lane];
    q0A = rt.qb0[lane];
  }
  if (lane + 64 < R) {
    nbB = rt.kblk_off[lane + 65] - rt.kblk_off[lane + 64];
    q0B = rt.qb0[lane + 64];
  }
  auto req = [&](int q, int& nb, int& q0) {
    nb = __builtin_amdgcn_readlane(q < 64 ? nbA : nbB, q & 63);
    q0 = __builtin_amdgcn_readlane(q < 64 ? q0A : q0B, q & 63);
  };
  int lo = 0, hi = rt.nb_max - 1;  // I lies in [lo, hi]; C(hi) = 0 <= pk
  while (lo < hi) {
    const int step = (hi - lo + 64) / 64;
    const int x = min(lo + (lane + 1) * step - 1, hi);  // lane 63 takes hi
    int cnt = 0;
    for (int q = 0; q < R; ++q) {
      int nb, q0;
      req(q, nb, q0);
      cnt += max(0, nb - max(x + 1, q0));
    }
    const uint64_t ok = __ballot(cnt <= pk);
    const int f = __builtin_ctzll(ok);
    hi = min(lo + (f + 1) * step - 1, hi);
    lo = lo + f * step;
  }
  I = lo;
  int j = pk;
  for (int q = 0; q < R; ++q) {
    int nb, q0;
    req(q, nb, q0);
    j -= max(0, nb - max(I + 1, q0));
  }
  r = 0;
  for (int q = 0; q < R; ++q) {
    int nb, q0;
    req(q, nb, q0);
    if (q0 <= I && nb > I) {
      if (j == 0) {
        r = q;
        break;
      }
      --j;
    }
  }
}

// blockIdx -> (key block I of a query block, request r) in descending-I order
// over the ragged batch, plus (kv head, sub-tile, split). Request r's query
// blocks are its key blocks qb0 .. NBk - 1 (all of them in a whole prefill).
__device__ __forceinline__ void decode_work(const AttnParams& p, int& I, int& r, int& h, int& sub, int& split) {
  const ReqTable& rt = p.rt;
  const int U = p.Hkv * p.subs * p.splits;
  const int pk = blockIdx.x / U;
  const int rem = blockIdx.x - pk * U;
  // Slot rem of the units of one query block runs on XCD rem % 8 (workgroups
  // go round-robin over the eight XCDs). Giving a slot the same KV head for
  // kRotateSpan / Hkv query blocks keeps that head's K / V tiles in one XCD's L2
  // across neighbouring rows; moving on afterwards spreads every head over
  // every XCD, so one head with more kept blocks does not hold back its XCD.
  h = (rem + pk / max(1, kRotateSpan / p.Hkv)) % p.Hkv;
  const int rem2 = rem / p.Hkv;
  sub = rem2 % p.subs;
  split = rem2 / p.subs;
  if (rt.R == 1) {
    // One request: its query blocks qb0 .. NBk - 1, heaviest first.
    r = 0;
    I = rt.kblk_off[1] - rt.kblk_off[0] - 1 - pk;
    return;
  }
  decode_multi(rt, pk, I, r);
}

// Starts the DMA of key block J of a row into one K tile and one V tile.
// Wave w, instruction u writes the 1 KiB group kWaves u + w of the tile:
// lane l fetches 16-byte chunk l/4 of tile row kSlab u + 4w + l%4 (FP8 K:
// chunk l/8 of row kSlab8 u + 8w + l%8).
template <int BLK, int PAGED, bool F8>
__device__ __forceinline__ void issue_block(const AttnParams& p, const RowCtx& rc, int J, uint8_t* kt, uint8_t* vt,
                                            int w, int lane, uint32_t voff_kv) {
  const int rstride = p.Hkv * kHeadDim * 2;  // bytes between consecutive tokens of bf16 K or V
  const int rs8 = p.Hkv * kHeadDim;          // the same for FP8 K
  const int lrem = rc.L - J * BLK;           // rows of block J inside the request (>= 1)
  if constexpr (!PAGED) {
    const int64_t tok0 = (rc.tok_base + (int64_t)J * BLK) * p.Hkv + rc.h;
    const uint8_t* kb = static_cast<const uint8_t*>(p.kk) + tok0 * (F8 ? kHeadDim : kHeadDim * 2);
    const uint8_t* vb = static_cast<const uint8_t*>(p.vv) + tok0 * (kHeadDim * 2);
    if constexpr (F8) {
      const uint32_t voff8 = (uint32_t)((8 * w + (lane & 7)) * rs8 + (lane >> 3) * 16);
#pragma unroll
      for (int u = 0; u < BLK / kSlab8; ++u) {
        const int nrec = uniform(min(max(lrem - kSlab8 * u, 0), kSlab8) * rs8);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(kb + (int64_t)(kSlab8 * u) * rs8, nrec),
                                                 (lds_ptr)(kt + (kWaves * u + w) * kOct), 16, voff8, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < BLK / kSlab; ++u) {
      const int nrec = uniform(min(max(lrem - kSlab * u, 0), kSlab) * rstride);
      const int64_t du = (int64_t)(kSlab * u) * rstride;
      if constexpr (!F8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(kb + du, nrec),
                                                 (lds_ptr)(kt + (kWaves * u + w) * kQuad), 16, voff_kv, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(vb + du, nrec),
                                               (lds_ptr)(vt + (kWaves * u + w) * kQuad), 16, voff_kv, 0, 0, 0);
    }
  } else {
    // Rows past the request repeat its last token (masked by the causal
    // mask of the diagonal item); each lane looks up its row's page.
    const int32_t* ptab = p.kv.page_table + (int64_t)rc.r * p.kv.max_pages;
    const int ps = p.kv.page_size;
    if constexpr (F8) {
#pragma unroll
      for (int u = 0; u < BLK / kSlab8; ++u) {
        const int t = J * BLK + min(kSlab8 * u + 8 * w + (lane & 7), lrem - 1);
        const int64_t off = (((int64_t)ptab[t / ps] * ps + t % ps) * p.Hkv + rc.h) * kHeadDim + (lane >> 3) * 16;
        __builtin_amdgcn_global_load_lds((gbl_ptr)(static_cast<const uint8_t*>(p.kk) + off),
                                         (lds_ptr)(kt + (kWaves * u + w) * kOct), 16, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < BLK / kSlab; ++u) {
      const int t = J * BLK + min(kSlab * u + 4 * w + (lane & 3), lrem - 1);
      const int64_t slot = ((int64_t)ptab[t / ps] * ps + t % ps) * p.Hkv + rc.h;
      const int64_t off = slot * (kHeadDim * 2) + (lane >> 2) * 16;
      if constexpr (!F8)
        __builtin_amdgcn_global_load_lds((gbl_ptr)(static_cast<const uint8_t*>(p.kk) + off),
                                         (lds_ptr)(kt + (kWaves * u + w) * kQuad), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_ptr)(static_cast<const uint8_t*>(p.vv) + off),
                                       (lds_ptr)(vt + (kWaves * u + w) * kQuad), 16, 0, 0);
    }
  }
}

// Key block of item e < n_exact of a row: item 0 is the diagonal block I,
// items 1 .. n_exact - 1 the CSR's other kept blocks in column order (the
// CSR row ends with the diagonal block, which is always kept).
__device__ __forceinline__ int item_block(const RowCtx& rc, const int32_t* colcache, int e) {
  if (e == 0) return rc.I;
  if (!rc.cols) return e - 1;
  return uniform(e - 1 < kColCache ? lload_i32(colcache + e - 1) : gload_i32(rc.cols + e - 1));
}

// Pruned blocks of a row: causal key blocks J < I whose bit in the row's
// selection bitmap is clear, one correction column each.

// Number of pruned blocks of row I (every lane of the wave gets it).
__device__ __forceinline__ int count_pruned(const uint32_t* selbits, int I, int lane) {
  const int nw = (I + 31) >> 5;
  int n = 0;
  for (int wd = lane; wd < nw; wd += 64) {
    uint32_t pm = ~selbits[wd];
    if (wd == (I >> 5)) pm &= (1u << (I & 31)) - 1u;
    n += __popc(pm);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) n += __shfl_xor(n, d);
  return n;
}

// The pruned blocks of row I in column order into plist (the caller ensures
// there are at most kPList). Wave w takes columns [w S, (w + 1) S), S a
// multiple of 64 with kWaves S >= I: its entries start at the number of
// pruned blocks before w S, and each round ranks 64 columns, one per lane,
// by a ballot.
__device__ __forceinline__ void list_pruned(const uint32_t* selbits, int I, int16_t* plist, int w, int lane) {
  const int S = (I + kWaves * 64 - 1) / (kWaves * 64) * 64;
  const int c0 = w * S, c1 = min(I, c0 + S);
  if (c0 >= c1) return;
  int at = 0;
  for (int wd = lane; wd < c0 / 32; wd += 64) at += __popc(~selbits[wd]);  // words wholly below c0 < I
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) at += __shfl_xor(at, d);
  for (int J = c0; J < c1; J += 64) {
    const int Jl = J + lane;
    const int Jc = min(Jl, c1 - 1);
    const bool pr = Jl < c1 && !((selbits[Jc >> 5] >> (Jc & 31)) & 1u);
    const uint64_t m = __ballot(pr);
    if (pr)
      plist[at + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] =
          (int16_t)Jl;
    at += __popcll(m);
  }
}

// Block of column t of correction chunk x: with the list, the pruned block of
// rank kPC x + t; else column kPC x + t if pruned (chunk x then spans key
// blocks kPC x .. kPC x + kPC - 1). -1: none (past the last, or selected).
__device__ __forceinline__ int chunk_block(const RowCtx& rc, const uint32_t* selbits, const int16_t* plist, int x,
                                           int t) {
  const int k = x * kPC + t;
  if (rc.listed) return k < rc.n_corr ? (int)plist[k] : -1;
  return k < rc.I && !((selbits[k >> 5] >> (k & 31)) & 1u) ? k : -1;
}

// Starts the DMA of item e into one K tile, one V tile and (pooled items) one
// bias row. A correction chunk gathers the bf16 pooled rows (256 bytes each)
// of its blocks; columns without one read zeros (an offset past the range)
// and get bias -inf.
template <int BLK, int PAGED, bool F8>
__device__ __forceinline__ void issue_item(const AttnParams& p, const RowCtx& rc, const int32_t* colcache,
                                           const uint32_t* selbits, const int16_t* plist, int e, uint8_t* kt,
                                           uint8_t* vt, float* bias, int tid, int w, int lane, uint32_t voff_kv) {
  if (e < rc.n_exact) {
    issue_block<BLK, PAGED, F8>(p, rc, item_block(rc, colcache, e), kt, vt, w, lane, voff_kv);
  } else {
    const int x = e - rc.n_exact;
    const int64_t row0 = rc.pooled_row0 * (kHeadDim * 2);
    const int nrec = rc.I * (kHeadDim * 2);
    const __amdgpu_buffer_rsrc_t kr = raw_rsrc(reinterpret_cast<const uint8_t*>(p.kbar16) + row0, nrec);
    const __amdgpu_buffer_rsrc_t vr = raw_rsrc(reinterpret_cast<const uint8_t*>(p.vbar16) + row0, nrec);
#pragma unroll
    for (int u = 0; u < kPC / kSlab; ++u) {
      const int J = chunk_block(rc, selbits, plist, x, kSlab * u + 4 * w + (lane & 3));
      const uint32_t off = J >= 0 ? (uint32_t)(J * (kHeadDim * 2) + (lane >> 2) * 16) : (uint32_t)nrec;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_ptr)(kt + (kWaves * u + w) * kQuad), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_ptr)(vt + (kWaves * u + w) * kQuad), 16, off, 0, 0, 0);
    }
    if (tid < kPC) {
      const int J = chunk_block(rc, selbits, plist, x, tid);
      bias[tid] = J >= 0 ? __log2f((float)min(BLK, rc.L - J * BLK)) : -INFINITY;
    }
  }
}

// Count-balanced split of a row's items: exact items (the first n_exact)
// cost 2, correction chunks 1; split s of S takes the items whose cost
// prefix starts in [s C / S, (s+1) C / S), C the row's total cost.
__device__ __forceinline__ int item_at_cost(int n_exact, int n_items, int64_t t) {
  // first item whose cost prefix is >= t
  if (t <= 2 * (int64_t)n_exact) return (int)((t + 1) / 2);
  return (int)min((int64_t)n_items, n_exact + (t - 2 * (int64_t)n_exact));
}

__device__ __forceinline__ void split_range(int n_exact, int n_items, int s, int S, int& e0, int& e1) {
  const int64_t C = 2 * (int64_t)n_exact + (n_items - n_exact);
  e0 = item_at_cost(n_exact, n_items, C * s / S);
  e1 = item_at_cost(n_exact, n_items, C * (s + 1) / S);
}

// Waits for this wave's tile DMA, then for every wave of the workgroup.
__device__ __forceinline__ void tiles_ready() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt unconstrained
  __syncthreads();
}

// One item of the row from tile set (kt, vt, bias).
template <int BLK, bool EXACT, bool F8>
__device__ __forceinline__ void compute_item(WaveState<BLK>& ws, const RowCtx& rc, int e, const uint8_t* kt,
                                             const uint8_t* vt, const float* bias, int tq0, int tq, float sl2,
                                             int lk, int lk8, int lv, int hf) {
  const int kind =
      EXACT ? kExact : (e == 0 ? (F8 && rc.I == 0 ? kDiagFirst : kDiag) : (e < rc.n_exact ? kExact : kPooled));
  attend_item<BLK, EXACT, F8>(ws, kt, vt, bias, kind, tq0 >> 5, tq, sl2, lk, lk8, lv, hf);
}

// PV of one half interleaved with QK^T of the next: the two MFMA streams
// alternate, so every accumulation chain sees at least three independent
// MFMAs between its own steps.
template <int DEPTH>
__device__ __forceinline__ void pv_qk_half(f32x16 (&o)[kHeadDim / 32], bf16x8 (&vf)[DEPTH], const bf16x8 (&pf)[2][2],
                                           const uint8_t* vh, const bf16x8 (&qf)[kHeadDim / 16], const uint8_t* kn,
                                           f32x16 (&sn)[2]) {
  constexpr int NJ = 16;
  bf16x8 kf[DEPTH];
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) kf[j] = k_operand<false>(kn, j);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    o[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j % DEPTH], pf[j >> 3][(j >> 2) & 1], o[j & 3], 0, 0, 0);
    if (j + DEPTH < NJ) vf[j % DEPTH] = v_operand(vh, j + DEPTH);
    sn[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j % DEPTH], qf[j >> 1], j < 2 ? f32x16{} : sn[j & 1], 0, 0, 0);
    if (j + DEPTH < NJ) kf[j % DEPTH] = k_operand<false>(kn, j + DEPTH);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// pv_qk_half with the next half's QK^T in FP8: one FP8 MFMA (twice the
// cycles of a bf16 one) after every fourth PV MFMA.
template <int DEPTH>
__device__ __forceinline__ void pv_qk_half8(f32x16 (&o)[kHeadDim / 32], bf16x8 (&vf)[DEPTH], const bf16x8 (&pf)[2][2],
                                            const uint8_t* vh, const i32x8 (&q8)[kHeadDim / 64], const uint8_t* kn,
                                            f32x16 (&sn)[2]) {
  constexpr int NJ = 16;
  i32x8 kf[2] = {k8_operand(kn, 0), k8_operand(kn, 1)};
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    o[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j % DEPTH], pf[j >> 3][(j >> 2) & 1], o[j & 3], 0, 0, 0);
    if (j + DEPTH < NJ) vf[j % DEPTH] = v_operand(vh, j + DEPTH);
    if ((j & 3) == 3) {
      const int q = j >> 2;
      sn[q & 1] = mfma_f8(kf[q & 1], q8[q >> 1], q < 2 ? f32x16{} : sn[q & 1]);
      if (q < 2) kf[q & 1] = k8_operand(kn, q + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Bytes between the K operands of consecutive halves (two 32-row tiles).
template <bool F8>
constexpr int kHalfK = F8 ? 8 * kOct : 16 * kQuad;

// Softmax and PV of half hh of a kept block whose scores are in sb[hh & 1],
// with the next half's QK^T interleaved into the PV.
template <int BLK, bool F8>
__device__ __forceinline__ void exact_halves(WaveState<BLK>& ws, const uint8_t* kh, const uint8_t* vt, float sl2,
                                             int lv, f32x16 (&sb)[2][2]) {
  constexpr int NH = BLK / 64;
  constexpr int kDepth = 4;
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    const uint8_t* vh = vt + lv + (2 * hh) * 8 * kQuad;
    bf16x8 vf[kDepth];
#pragma unroll
    for (int j = 0; j < kDepth; ++j) vf[j] = v_operand(vh, j);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 pf[2][2];
    softmax_half(ws, sb[hh & 1], sl2, pf);
    __builtin_amdgcn_sched_barrier(0);
    if (hh + 1 < NH) {
      if constexpr (F8)
        pv_qk_half8<kDepth>(ws.o, vf, pf, vh, ws.q8, kh + (hh + 1) * kHalfK<F8>, sb[(hh + 1) & 1]);
      else
        pv_qk_half<kDepth>(ws.o, vf, pf, vh, ws.qf, kh + (hh + 1) * kHalfK<F8>, sb[(hh + 1) & 1]);
    } else {
      pv_jobs<16, kDepth>(ws.o, vf, pf, vh);
    }
  }
}

// An off-diagonal kept block: all keys visible, no score adjustment. Its
// halves are software-pipelined: QK^T(0); softmax(0); PV(0) with QK^T(1);
// softmax(1); PV(1). kh: the lane's K operand base in the tile.
template <int BLK, bool F8>
__device__ __forceinline__ void attend_exact(WaveState<BLK>& ws, const uint8_t* kh, const uint8_t* vt, float sl2,
                                             int lv) {
  f32x16 sb[2][2];
  if constexpr (F8)
    qk_half8(ws.q8, kh, sb[0]);
  else
    qk_half<4, false>(ws.qf, kh, sb[0]);
  exact_halves<BLK, F8>(ws, kh, vt, sl2, lv, sb);
}

// The next kept block's K / V DMA (BLK rows in 32-row slabs, K and V each),
// prepared after the item barrier and issued one instruction per MFMA during
// the first QK^T half, so the eight waves do not all stall together while
// the vector memory unit accepts them (contiguous K / V only).
struct ItemDma {
  static constexpr int kFirst = 0;  // MFMA after which instruction 0 goes out
  const uint8_t* kb;
  const uint8_t* vb;
  int lrem;  // rows of the block inside the request
  int rstride;
  uint32_t voff;
  uint8_t* kt;
  uint8_t* vt;
  int w;
  // Instruction I: K (I even) or V (I odd) of slab I / 2.
  template <int I>
  __device__ __forceinline__ void fire() const {
    constexpr int u = I >> 1;
    const int nrec = uniform(min(max(lrem - kSlab * u, 0), kSlab) * rstride);
    const int64_t du = (int64_t)(kSlab * u) * rstride;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(((I & 1) ? vb : kb) + du, nrec),
                                             (lds_ptr)(((I & 1) ? vt : kt) + (kWaves * u + w) * kQuad), 16, voff,
                                             0, 0, 0);
  }
};

template <int BLK>
__device__ __forceinline__ ItemDma prep_block(const AttnParams& p, const RowCtx& rc, const int32_t* colcache, int e,
                                              uint8_t* kt, uint8_t* vt, int w, uint32_t voff_kv) {
  const int J = item_block(rc, colcache, e);
  const int64_t row0 = ((rc.tok_base + (int64_t)J * BLK) * p.Hkv + rc.h) * (kHeadDim * 2);
  ItemDma d;
  d.kb = static_cast<const uint8_t*>(p.kk) + row0;
  d.vb = static_cast<const uint8_t*>(p.vv) + row0;
  d.lrem = rc.L - J * BLK;
  d.rstride = p.Hkv * kHeadDim * 2;
  d.voff = voff_kv;
  d.kt = kt;
  d.vt = vt;
  d.w = w;
  return d;
}

// The next kept block's DMA in paged K / V, for page sizes that are a
// multiple of 4: the four rows one wave's instruction fills (4w .. 4w+3 of a
// 32-row slab, 4-aligned) then lie in one page, so each slab needs one page
// id per wave, read by a scalar load when the DMA is prepared, and the
// instruction reads the rows through a buffer range from that page's row
// (rows past the request read zeros, masked as keys past every query). Its
// instructions go out from the fifth MFMA on, leaving the page loads time.
struct PagedDma {
  static constexpr int kFirst = 4;
  const uint8_t* kk;
  const uint8_t* vv;
  int64_t off[4];  // byte offset of the wave's first row of slab u (K and V alike)
  int nrec[4];     // bytes of that 4-row group inside the request
  uint32_t voff;   // lane: row lane % 4 of the group, chunk lane / 4
  uint8_t* kt;
  uint8_t* vt;
  int w;
  template <int I>
  __device__ __forceinline__ void fire() const {
    constexpr int u = I >> 1;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(((I & 1) ? vv : kk) + off[u], nrec[u]),
                                             (lds_ptr)(((I & 1) ? vt : kt) + (kWaves * u + w) * kQuad), 16, voff,
                                             0, 0, 0);
  }
};

template <int BLK>
__device__ __forceinline__ PagedDma prep_paged(const AttnParams& p, const RowCtx& rc, const int32_t* colcache, int e,
                                               uint8_t* kt, uint8_t* vt, int w, int lane) {
  static_assert(BLK / kSlab <= 4, "slabs per block");
  const int J = item_block(rc, colcache, e);
  const int lrem = rc.L - J * BLK;
  const int rstride = p.Hkv * kHeadDim * 2;
  PagedDma d;
  d.kk = static_cast<const uint8_t*>(p.kk);
  d.vv = static_cast<const uint8_t*>(p.vv);
  d.voff = (uint32_t)((lane & 3) * rstride + (lane >> 2) * 16);
  d.kt = kt;
  d.vt = vt;
  d.w = w;
  const int32_t* ptab = p.kv.page_table + (int64_t)rc.r * p.kv.max_pages;
#pragma unroll
  for (int u = 0; u < BLK / kSlab; ++u) {
    const int r0 = kSlab * u + 4 * w;  // the wave's first row of the slab
    const int t = J * BLK + min(r0, lrem - 1);
    const int page = sload_i32(ptab + t / p.kv.page_size);
    d.off[u] = (((int64_t)page * p.kv.page_size + t % p.kv.page_size) * p.Hkv + rc.h) * (kHeadDim * 2);
    d.nrec[u] = uniform(min(max(lrem - r0, 0), 4) * rstride);
  }
  return d;
}

// qk_half with a block's DMA spread over its first MFMAs (two per slab).
template <int DEPTH, int BLK, typename D>
__device__ __forceinline__ void qk_half_dma(const bf16x8 (&qf)[kHeadDim / 16], const uint8_t* kh, f32x16 (&s)[2],
                                            const D& d) {
  constexpr int NJ = 2 * (kHeadDim / 16);
  constexpr int NF = 2 * (BLK / kSlab);
  bf16x8 kf[DEPTH];
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) kf[j] = k_operand<false>(kh, j);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    s[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j % DEPTH], qf[j >> 1], j < 2 ? f32x16{} : s[j & 1], 0, 0, 0);
    if (j + DEPTH < NJ) kf[j % DEPTH] = k_operand<false>(kh, j + DEPTH);
    if constexpr (NF > 0) if (j == D::kFirst + 0) d.template fire<0>();
    if constexpr (NF > 1) if (j == D::kFirst + 1) d.template fire<1>();
    if constexpr (NF > 2) if (j == D::kFirst + 2) d.template fire<2>();
    if constexpr (NF > 3) if (j == D::kFirst + 3) d.template fire<3>();
    if constexpr (NF > 4) if (j == D::kFirst + 4) d.template fire<4>();
    if constexpr (NF > 5) if (j == D::kFirst + 5) d.template fire<5>();
    if constexpr (NF > 6) if (j == D::kFirst + 6) d.template fire<6>();
    if constexpr (NF > 7) if (j == D::kFirst + 7) d.template fire<7>();
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The next kept block's DMA for FP8 K (contiguous K / V): the BLK / 64 FP8
// K instructions, then the bf16 V slabs.
template <int BLK>
struct ItemDma8 {
  static constexpr int kNK = BLK / kSlab8;
  static constexpr int kCount = kNK + BLK / kSlab;
  const uint8_t* kb;  // FP8 K rows of the block (row stride rstride / 2)
  const uint8_t* vb;  // bf16 V rows
  int lrem;
  int rstride;
  uint32_t voff, voff8;
  uint8_t* kt;
  uint8_t* vt;
  int w;
  template <int I>
  __device__ __forceinline__ void fire() const {
    if constexpr (I < kNK) {
      const int rs8 = rstride >> 1;
      const int nrec = uniform(min(max(lrem - kSlab8 * I, 0), kSlab8) * rs8);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(kb + (int64_t)(kSlab8 * I) * rs8, nrec),
                                               (lds_ptr)(kt + (kWaves * I + w) * kOct), 16, voff8, 0, 0, 0);
    } else {
      constexpr int u = I - kNK;
      const int nrec = uniform(min(max(lrem - kSlab * u, 0), kSlab) * rstride);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(vb + (int64_t)(kSlab * u) * rstride, nrec),
                                               (lds_ptr)(vt + (kWaves * u + w) * kQuad), 16, voff, 0, 0, 0);
    }
  }
};

template <int BLK>
__device__ __forceinline__ ItemDma8<BLK> prep_block8(const AttnParams& p, const RowCtx& rc, const int32_t* colcache,
                                                     int e, uint8_t* kt, uint8_t* vt, int w, int lane,
                                                     uint32_t voff_kv) {
  const int J = item_block(rc, colcache, e);
  const int64_t tok0 = (rc.tok_base + (int64_t)J * BLK) * p.Hkv + rc.h;
  ItemDma8<BLK> d;
  d.kb = static_cast<const uint8_t*>(p.kk) + tok0 * kHeadDim;
  d.vb = static_cast<const uint8_t*>(p.vv) + tok0 * (kHeadDim * 2);
  d.lrem = rc.L - J * BLK;
  d.rstride = p.Hkv * kHeadDim * 2;
  d.voff = voff_kv;
  d.voff8 = (uint32_t)((8 * w + (lane & 7)) * (p.Hkv * kHeadDim) + (lane >> 3) * 16);
  d.kt = kt;
  d.vt = vt;
  d.w = w;
  return d;
}

// Issues DMA instructions [0, NF) of d.
template <int NF, typename D>
__device__ __forceinline__ void fire_all(const D& d) {
  if constexpr (NF > 0) d.template fire<0>();
  if constexpr (NF > 1) d.template fire<1>();
  if constexpr (NF > 2) d.template fire<2>();
  if constexpr (NF > 3) d.template fire<3>();
  if constexpr (NF > 4) d.template fire<4>();
  if constexpr (NF > 5) d.template fire<5>();
  if constexpr (NF > 6) d.template fire<6>();
  if constexpr (NF > 7) d.template fire<7>();
}

// qk_half8 with a block's DMA spread over its MFMAs, two instructions after
// each (an FP8 MFMA takes as long as two bf16 ones).
template <int BLK>
__device__ __forceinline__ void qk_half8_dma(const i32x8 (&q8)[kHeadDim / 64], const uint8_t* kh, f32x16 (&s)[2],
                                             const ItemDma8<BLK>& d) {
  constexpr int NF = ItemDma8<BLK>::kCount;
  static_assert(NF <= 8, "two DMA instructions per FP8 MFMA");
  i32x8 kf[2] = {k8_operand(kh, 0), k8_operand(kh, 1)};
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    s[j & 1] = mfma_f8(kf[j & 1], q8[j >> 1], j < 2 ? f32x16{} : s[j & 1]);
    if (j < 2) kf[j & 1] = k8_operand(kh, j + 2);
    if constexpr (NF > 0) if (j == 0) d.template fire<0>();
    if constexpr (NF > 1) if (j == 0) d.template fire<1>();
    if constexpr (NF > 2) if (j == 1) d.template fire<2>();
    if constexpr (NF > 3) if (j == 1) d.template fire<3>();
    if constexpr (NF > 4) if (j == 2) d.template fire<4>();
    if constexpr (NF > 5) if (j == 2) d.template fire<5>();
    if constexpr (NF > 6) if (j == 3) d.template fire<6>();
    if constexpr (NF > 7) if (j == 3) d.template fire<7>();
    __builtin_amdgcn_sched_barrier(0);
  }
}

// attend_exact whose first QK^T half also issues the next block's DMA.
template <int BLK, bool F8, typename D>
__device__ __forceinline__ void attend_exact_dma(WaveState<BLK>& ws, const uint8_t* kh, const uint8_t* vt, float sl2,
                                                 int lv, const D& d) {
  f32x16 sb[2][2];
  if constexpr (F8)
    qk_half8_dma<BLK>(ws.q8, kh, sb[0], d);
  else
    qk_half_dma<4, BLK, D>(ws.qf, kh, sb[0], d);
  exact_halves<BLK, F8>(ws, kh, vt, sl2, lv, sb);
}

// The item loop of one workgroup. step<EXACT, SET>: stream item e+1 into the
// other tile set while item e is computed from set SET, then wait for the
// stream and for every wave.
template <int BLK, int PAGED, bool F8>
struct ItemLoop {
  const AttnParams& p;
  const RowCtx& rc;
  const int32_t* colcache;
  const uint32_t* selbits;
  const int16_t* plist;
  uint8_t *kt0, *kt1, *vt0, *vt1;
  float *bias0, *bias1;
  int N, tid, w, lane;
  uint32_t voff_kv;
  bool wave_active;
  int tq0, tq;
  float sl2;
  int lk, lk8, lv, hf;
  // The lane's K operand base for kept blocks.
  __device__ __forceinline__ int lkx() const { return F8 ? lk8 : lk; }

  // A kept block from tile set `set`, with the next block's DMA D (NF
  // instructions) spread over its first QK^T half.
  template <int NF, typename D>
  __device__ __forceinline__ void spread_step(WaveState<BLK>& ws, const D& d, int set) {
    if (wave_active)
      attend_exact_dma<BLK, F8, D>(ws, (set ? kt1 : kt0) + lkx(), set ? vt1 : vt0, sl2, lv, d);
    else
      fire_all<NF>(d);
  }

  template <bool EXACT, int SET>
  __device__ __forceinline__ void step(WaveState<BLK>& ws, int e) {
    if constexpr (EXACT) {
      // The next item is an off-diagonal or the diagonal block: its DMA runs
      // inside this item's first QK^T half (waves without rows issue it here).
      // Paged K / V with a page size that is not a multiple of 4 (and
      // paged FP8 K, whose 8-row groups may straddle pages) keeps the burst
      // below.
      if constexpr (F8 && PAGED == kContig) {
        const ItemDma8<BLK> d =
            prep_block8<BLK>(p, rc, colcache, e + 1, SET ? kt0 : kt1, SET ? vt0 : vt1, w, lane, voff_kv);
        spread_step<ItemDma8<BLK>::kCount>(ws, d, SET);
        tiles_ready();
        return;
      } else if constexpr (!F8 && PAGED != kPagedAny) {
        if constexpr (PAGED) {
          const PagedDma d = prep_paged<BLK>(p, rc, colcache, e + 1, SET ? kt0 : kt1, SET ? vt0 : vt1, w, lane);
          spread_step<2 * (BLK / kSlab)>(ws, d, SET);
        } else {
          const ItemDma d = prep_block<BLK>(p, rc, colcache, e + 1, SET ? kt0 : kt1, SET ? vt0 : vt1, w, voff_kv);
          spread_step<2 * (BLK / kSlab)>(ws, d, SET);
        }
        tiles_ready();
        return;
      }
    }
    if (e + 1 < N)
      issue_item<BLK, PAGED, F8>(p, rc, colcache, selbits, plist, e + 1, SET ? kt0 : kt1, SET ? vt0 : vt1,
                                 SET ? bias0 : bias1, tid, w, lane, voff_kv);
    if (wave_active) {
      if (EXACT)
        attend_exact<BLK, F8>(ws, (SET ? kt1 : kt0) + lkx(), SET ? vt1 : vt0, sl2, lv);
      else
        compute_item<BLK, false, F8>(ws, rc, e, SET ? kt1 : kt0, SET ? vt1 : vt0, SET ? bias1 : bias0, tq0, tq,
                                     sl2, lk, lk8, lv, hf);
    }
    tiles_ready();
  }

  template <bool EXACT>
  __device__ __forceinline__ void run(WaveState<BLK>& ws, int e0, int e1) {
    int e = e0;
    if (e < e1 && (e & 1)) step<EXACT, 1>(ws, e++);
    for (; e + 1 < e1; e += 2) {
      step<EXACT, 0>(ws, e);
      step<EXACT, 1>(ws, e + 1);
    }
    if (e < e1) step<EXACT, 0>(ws, e);
  }
};

// F8: Q and K are E4M3 codes (QK^T on the FP8 matrix cores), V a bf16 copy
// of its codes. DENSE only names the instantiation the dense comparator
// (p.dense) launches, so that a kernel trace keeps its dispatches apart from
// the sparse launches'; the code does not read it.
template <int BLK, int PAGED, bool SPLIT, bool F8, bool DENSE>
__global__ __launch_bounds__(kThreads, 1) void attn_kernel(AttnParams p) {
  // Two tile sets, each its own LDS object, so the compiler can tell the
  // in-flight DMA into one set from the operand reads of the other.
  __shared__ uint4 k_lds0[Tile<BLK>::kWords], k_lds1[Tile<BLK>::kWords];
  __shared__ uint4 v_lds0[Tile<BLK>::kWords], v_lds1[Tile<BLK>::kWords];
  __shared__ float bias0[kPC], bias1[kPC];
  __shared__ uint32_t selbits[FP_MAX_BLOCKS_PER_SEQ / 32];
  __shared__ int32_t colcache[kColCache];
  __shared__ int16_t plist[kPList];
  uint8_t* const kt0 = reinterpret_cast<uint8_t*>(k_lds0);
  uint8_t* const kt1 = reinterpret_cast<uint8_t*>(k_lds1);
  uint8_t* const vt0 = reinterpret_cast<uint8_t*>(v_lds0);
  uint8_t* const vt1 = reinterpret_cast<uint8_t*>(v_lds1);

  RowCtx rc;
  int sub, split;
  decode_work(p, rc.I, rc.r, rc.h, sub, split);
  const ReqTable& rt = p.rt;
  rc.tok_base = rt.ktok_off[rc.r];
  rc.L = rt.ktok_off[rc.r + 1] - rt.ktok_off[rc.r];
  const int I = rc.I;
  const int qi = I - rt.qb0[rc.r];  // query block of the call
  const int nI = min(BLK, rc.L - I * BLK);
  const int64_t row = (int64_t)rc.h * p.NBq_tot + rt.blk_off[rc.r] + qi;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  // Waves w and w + 4 share a SIMD. The first of each pair keeps a higher
  // issue priority for the whole kernel, so after each item barrier it takes
  // the matrix core first and the pair drifts apart: one wave's softmax then
  // runs under the other's MFMAs instead of both stalling on the same phase.
  if (w < 4) __builtin_amdgcn_s_setprio(3);
  const int c = lane & 31, hf = lane >> 5;
  const int prow0 = sub * kRowsPerWG + w * 32;  // first packed row of this wave
  const bool wave_active = prow0 < p.G * BLK;
  const int g = rc.h * p.G + (wave_active ? prow0 / BLK : 0);
  const int tq0 = prow0 % BLK;
  const int tq = tq0 + c;
  const bool q_valid = wave_active && tq < nI;
  const int64_t tok = rt.tok_off[rc.r] + (int64_t)qi * BLK + tq;  // query token
  // K operand: row c of a 32-row tile, chunk hf (then + 128 bytes per 16
  // dims); with FP8 Q (correction chunks) chunk 4 hf, see k_operand. FP8 K:
  // row c, chunk 2 hf (then + 512 bytes per 64 dims).
  const int lk = (c >> 2) * kQuad + (c & 3) * 16 + hf * (F8 ? 256 : 64);
  const int lk8 = (c >> 3) * kOct + (c & 7) * 16 + hf * 256;
  // V^T operand: lane j of 16-lane group gq reads dims 16(gq&1) + 4(j&3)..+3 of
  // key 4(gq>>1) + j/4 (tile_off layout).
  const int j16 = lane & 15, gq = lane >> 4;
  const int lv = (gq >> 1) * kQuad + (gq & 1) * 128 + ((j16 & 3) >> 1) * 64 + (j16 >> 2) * 16 + (j16 & 1) * 8;
  // DMA offsets: chunk lane/4 of row 4w + lane%4 of a 32-row slab.
  const uint32_t voff_kv = (uint32_t)((4 * w + (lane & 3)) * p.Hkv * kHeadDim * 2 + (lane >> 2) * 16);

  // Logit scale in log2 units. FP8 folds the Q and K descales into it (K, V
  // and the pooled rows are staged in code units) and multiplies the output
  // by the V descale.
  float sl2 = p.sm_scale * kLog2e;
  float oscale = 1.f;
  if constexpr (F8) {
    sl2 *= *p.descale_q * *p.descale_k;
    oscale = *p.descale_v;
  }

  // Q rows of a bf16 unsplit launch with 128-key blocks are staged through
  // the idle tile set 1 by DMA, 16 lanes per 256-byte row, so each load
  // instruction reads four whole rows; loading the operands directly would
  // touch 32 rows (lines) per instruction, each four times. Wave w stages
  // its 32 rows in groups of four, kQGroup bytes apart (the padding spreads
  // the operand reads over the banks).
  // Without split-KV the row starts at item 0, the diagonal block: it needs
  // no CSR entry, so its DMA starts first, while Q and the row's tables load.
  if constexpr (!SPLIT) issue_block<BLK, PAGED, F8>(p, rc, I, kt0, vt0, w, lane, voff_kv);

  constexpr int kQGroup = 4 * kHeadDim * 2 + 16;
  constexpr bool kQStage = BLK == 128 && !SPLIT;
  static_assert(!kQStage || 4 * 8 * kQGroup <= (int)(Tile<BLK>::kWords * 16), "Q staging space");
  constexpr bool q_lds = kQStage && !F8;
  uint8_t* const qs = ((w >> 2) ? vt1 : kt1) + (w & 3) * 8 * kQGroup;
  if (q_lds && wave_active) {
    const int nvalid = max(0, min(32, nI - tq0));  // rows of the wave's 32 that exist
    const int rstride = p.Hq * kHeadDim * 2;
    const uint8_t* qb = static_cast<const uint8_t*>(p.q) + ((tok - c) * p.Hq + g) * (kHeadDim * 2);
    const uint32_t qoff = (uint32_t)((lane >> 4) * rstride + (lane & 15) * 16);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      // Buffer range: rows 4 it .. nvalid - 1 (bytes past the base of row 4 it).
      const int nrec = uniform(nvalid > 4 * it ? (nvalid - 1 - 4 * it) * rstride + kHeadDim * 2 : 0);
      // Non-temporal (aux 2): the rows are read by this workgroup only, so
      // they need not displace the kept K/V tiles that other rows reuse from
      // L2 and MALL.
      __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(qb + (int64_t)(4 * it) * rstride, nrec),
                                               (lds_ptr)(qs + it * kQGroup), 16, qoff, 0, 0, 2);
    }
  }

  // The row's CSR extent (scalar loads, after the DMA above so they do not
  // delay it).
  const int rp0 = p.dense ? 0 : sload_i32(p.row_ptr + row);
  rc.n_exact = p.dense ? I + 1 : sload_i32(p.row_ptr + row + 1) - rp0;
  rc.cols = p.dense ? nullptr : p.col_idx + rp0;
  const bool do_corr = p.mean_correction && !p.dense && I > 0;
  rc.pooled_row0 = (int64_t)rc.h * p.kpitch + rt.prow_off[rc.r];

  WaveState<BLK> ws;
  ws.m = kNegBig;
  ws.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < kHeadDim / 32; ++dt) ws.o[dt] = f32x16{};
  if constexpr (F8) {
    // Lane (c, hf): codes 64 ks2 + 32 hf .. + 31 of its query.
#pragma unroll
    for (int ks2 = 0; ks2 < kHeadDim / 64; ++ks2) {
      uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
      if (q_valid) {
        const uint8_t* qp = static_cast<const uint8_t*>(p.q) + (tok * p.Hq + g) * kHeadDim + ks2 * 64 + hf * 32;
        a = *reinterpret_cast<const uint4*>(qp);
        b = *reinterpret_cast<const uint4*>(qp + 16);
      }
      ws.q8[ks2] = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    }
  } else if (!q_lds) {
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 16; ++ks) {
      uint4 qv = make_uint4(0, 0, 0, 0);
      if (q_valid)
        qv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + (tok * p.Hq + g) * kHeadDim +
                                             ks * 16 + hf * 8);
      ws.qf[ks] = __builtin_bit_cast(bf16x8, qv);
    }
  }

  if (!p.dense) {
    if (do_corr)
      for (int wd = tid; wd <= (I >> 5); wd += kThreads) selbits[wd] = 0u;
    for (int e = tid; e < min(rc.n_exact, kColCache); e += kThreads) colcache[e] = rc.cols[e];
  }
  if constexpr (q_lds) {
    // This wave's staged rows have landed (with the block and the columns):
    // lane (c, hf) takes 16-byte chunk 2 ks + hf of row c.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    const uint8_t* qr = qs + (c >> 2) * kQGroup + (c & 3) * (kHeadDim * 2) + hf * 16;
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 16; ++ks) ws.qf[ks] = *reinterpret_cast<const bf16x8*>(qr + ks * 32);
  }
  if (!p.dense) {
    __syncthreads();
    if (do_corr) {
      for (int e = tid; e < rc.n_exact; e += kThreads) {
        const int J = e < kColCache ? lload_i32(colcache + e) : gload_i32(rc.cols + e);
        atomicOr(&selbits[J >> 5], 1u << (J & 31));
      }
    }
    __syncthreads();
  }
  // Correction chunks: the row's pruned blocks, kPC per chunk, from a list
  // the waves build now (the next barrier publishes it); a row with more
  // than kPList of them takes its chunks over consecutive key blocks instead.
  rc.n_corr = do_corr ? uniform(count_pruned(selbits, I, lane)) : 0;
  rc.listed = rc.n_corr <= kPList;
  if (rc.listed && rc.n_corr > 0) list_pruned(selbits, I, plist, w, lane);
  rc.n_items = rc.n_exact + (rc.listed ? (rc.n_corr + kPC - 1) / kPC : (I + kPC - 1) / kPC);

  // Items [e0, e1) of this split (all items without split-KV): the diagonal
  // block, the other kept blocks, the correction chunks. The kept blocks
  // between the first and the last run through an instantiation of the item
  // code without any score adjustment (its DMA step can only stream a block
  // next); the others through the general one. Item e always lives in tile
  // set e & 1.
  if constexpr (SPLIT) {
    int e0, e1;
    split_range(rc.n_exact, rc.n_items, split, p.splits, e0, e1);
    if (e0 < e1) {
      if (e0 >= rc.n_exact) __syncthreads();  // the list, for the first item
      const bool odd = e0 & 1;
      issue_item<BLK, PAGED, F8>(p, rc, colcache, selbits, plist, e0, odd ? kt1 : kt0, odd ? vt1 : vt0,
                                 odd ? bias1 : bias0, tid, w, lane, voff_kv);
      tiles_ready();
      ItemLoop<BLK, PAGED, F8> L{p, rc, colcache, selbits, plist, kt0, kt1, vt0, vt1, bias0, bias1, e1, tid, w,
                                 lane, voff_kv, wave_active, tq0, tq, sl2, lk, lk8, lv, hf};
      L.template run<false>(ws, e0, min(e1, 1));
      L.template run<true>(ws, max(e0, 1), min(e1, rc.n_exact - 1));
      L.template run<false>(ws, max(e0, max(1, rc.n_exact - 1)), e1);
    }
  } else {
    const int N = rc.n_items;
    tiles_ready();
    ItemLoop<BLK, PAGED, F8> L{p, rc, colcache, selbits, plist, kt0, kt1, vt0, vt1, bias0, bias1, N, tid, w,
                               lane, voff_kv, wave_active, tq0, tq, sl2, lk, lk8, lv, hf};
    L.template run<false>(ws, 0, 1);
    L.template run<true>(ws, 1, rc.n_exact - 1);
    L.template run<false>(ws, max(1, rc.n_exact - 1), N);
  }

  if (!wave_active) return;
  const float l_tot = sum_halves(ws.l);
  if constexpr (SPLIT) {
    // Partial result of this split: o / l and log2(l) + m (-inf when the
    // split saw no key), in the workspace for merge_kernel.
    if (q_valid) {
      const int64_t prow = ((int64_t)split * p.T + tok) * p.Hq + g;
      const float inv = l_tot > 0.f ? oscale / l_tot : 0.f;
      float* orow = p.o_part + prow * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < kHeadDim / 32; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 v = make_float4(ws.o[dt][4 * i + 0] * inv, ws.o[dt][4 * i + 1] * inv,
                                       ws.o[dt][4 * i + 2] * inv, ws.o[dt][4 * i + 3] * inv);
          *reinterpret_cast<float4*>(orow + dt * 32 + i * 8 + hf * 4) = v;
        }
      }
      if (hf == 0) p.lse_part[prow] = l_tot > 0.f ? ws.m + __log2f(l_tot) : -INFINITY;
    }
    return;
  }
  // Output rows through LDS: a lane holds 8-byte pieces of its query's row,
  // and rows of one head lie Hq * 256 bytes apart, so direct stores would
  // write 64 partial lines per instruction. The wave stages its 32 rows in
  // its own part of the (now idle) tile buffers, 272 bytes apart, and stores
  // them back 16 lanes per row: whole 256-byte rows.
  {
    const float inv = q_valid ? oscale / l_tot : 0.f;
    constexpr int kOStride = kHeadDim * 2 + 16;
    constexpr int kOStage = 32 * kOStride;
    constexpr int kPer = (int)(Tile<BLK>::kWords * 16) / kOStage;  // waves per tile object
    static_assert(kPer * 4 >= kWaves, "staging space");
    const int oi = w / kPer;
    uint8_t* const st = (oi == 0 ? kt0 : oi == 1 ? kt1 : oi == 2 ? vt0 : vt1) + (w % kPer) * kOStage;
#pragma unroll
    for (int dt = 0; dt < kHeadDim / 32; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 pk;
        pk.x = pack_bf16x2(ws.o[dt][4 * i + 0] * inv, ws.o[dt][4 * i + 1] * inv);
        pk.y = pack_bf16x2(ws.o[dt][4 * i + 2] * inv, ws.o[dt][4 * i + 3] * inv);
        *reinterpret_cast<uint2*>(st + c * kOStride + (dt * 32 + i * 8 + hf * 4) * 2) = pk;
      }
    }
    const int64_t tok0 = tok - c;  // token of the wave's first row
    const int chunk = lane & 15;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int rr = 4 * it + (lane >> 4);
      const uint4 v = *reinterpret_cast<const uint4*>(st + rr * kOStride + chunk * 16);
      // Non-temporal: the output is written once and read by no kernel here.
      if (tq0 + rr < nI)
        __builtin_nontemporal_store(
            u32x4{v.x, v.y, v.z, v.w},
            reinterpret_cast<u32x4*>(p.out + ((tok0 + rr) * p.Hq + g) * kHeadDim + chunk * 8));
    }
  }
  if (q_valid && p.lse != nullptr && hf == 0) p.lse[(int64_t)g * p.T + tok] = (ws.m + __log2f(l_tot)) * kLn2;
}

// Conversion pass before the attention kernel (one launch, grid-stride):
// bf16 copies of k_bar, v_bar in code units (divided by the K / V descales
// for FP8), and for FP8 the V codes as bf16 (exact, two codes per
// v_cvt_scalef32_pk_bf16_fp8; K stays FP8).
__global__ __launch_bounds__(256) void prep_kernel(AttnParams p, int64_t n_pool8, int64_t n_kv8) {
  const float ks = p.fp8 ? 1.f / *p.descale_k : 1.f;
  const float vs = p.fp8 ? 1.f / *p.descale_v : 1.f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * n_pool8 + n_kv8; i += stride) {
    if (i < 2 * n_pool8) {
      const bool isv = i >= n_pool8;
      const int64_t k8 = isv ? i - n_pool8 : i;
      const float* src = (isv ? p.v_bar : p.k_bar) + k8 * 8;
      const float s = isv ? vs : ks;
      const float4 a = *reinterpret_cast<const float4*>(src);
      const float4 b = *reinterpret_cast<const float4*>(src + 4);
      uint4 o;
      o.x = pack_bf16x2(a.x * s, a.y * s);
      o.y = pack_bf16x2(a.z * s, a.w * s);
      o.z = pack_bf16x2(b.x * s, b.y * s);
      o.w = pack_bf16x2(b.z * s, b.w * s);
      reinterpret_cast<uint4*>(isv ? p.vbar16 : p.kbar16)[k8] = o;
    } else {
      const int64_t k8 = i - 2 * n_pool8;
      const uint2 c = reinterpret_cast<const uint2*>(p.v)[k8];
      const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, false);
      const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, true);
      const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, false);
      const bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, true);
      reinterpret_cast<bf16x8*>(const_cast<void*>(p.vv))[k8] = bf16x8{a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
    }
  }
}

// Split-KV merge: for each (query token, query head), the parts' log2-sum-
// exps L_s give weights 2^(L_s - M) / sum_s 2^(L_s - M); O is the weighted
// sum of the parts' normalised outputs (bf16 out) and LSE = (M + log2 of the
// weight sum) * ln 2. 32 lanes per row, four dims each.
__global__ __launch_bounds__(256) void merge_kernel(AttnParams p) {
  const int64_t rows = (int64_t)p.T * p.Hq;
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int c = (threadIdx.x & 31) * 4;
  if (row >= rows) return;
  float M = -INFINITY;
  for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.lse_part[(int64_t)s * rows + row]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  for (int s = 0; s < p.splits; ++s) {
    const float ls = p.lse_part[(int64_t)s * rows + row];
    if (ls == -INFINITY) continue;
    const float wgt = __builtin_amdgcn_exp2f(ls - M);
    const float4 o = *reinterpret_cast<const float4*>(p.o_part + ((int64_t)s * rows + row) * kHeadDim + c);
    acc.x = fmaf(wgt, o.x, acc.x);
    acc.y = fmaf(wgt, o.y, acc.y);
    acc.z = fmaf(wgt, o.z, acc.z);
    acc.w = fmaf(wgt, o.w, acc.w);
    wsum += wgt;
  }
  const float inv = 1.f / wsum;
  uint2 pk;
  pk.x = pack_bf16x2(acc.x * inv, acc.y * inv);
  pk.y = pack_bf16x2(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2*>(p.out + row * kHeadDim + c) = pk;
  if (p.lse != nullptr && c == 0) {
    const int64_t tok = row / p.Hq;
    const int g = (int)(row % p.Hq);
    p.lse[(int64_t)g * p.T + tok] = (M + __log2f(wsum)) * kLn2;
  }
}

template <int BLK, int PAGED, bool SPLIT, bool F8>
void launch_attn_v(const AttnParams& p, dim3 grid, hipStream_t stream) {
  if (p.dense)
    hipLaunchKernelGGL((attn_kernel<BLK, PAGED, SPLIT, F8, true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_kernel<BLK, PAGED, SPLIT, F8, false>), grid, dim3(kThreads), 0, stream, p);
}

template <int BLK, bool SPLIT>
void launch_attn_t(const AttnParams& p, dim3 grid, hipStream_t stream) {
  if (p.fp8) {
    if (!p.kv.paged) launch_attn_v<BLK, kContig, SPLIT, true>(p, grid, stream);
    else launch_attn_v<BLK, kPagedAny, SPLIT, true>(p, grid, stream);
  } else if (!p.kv.paged) {
    launch_attn_v<BLK, kContig, SPLIT, false>(p, grid, stream);
  } else if (p.kv.page_size % 4 == 0) {
    launch_attn_v<BLK, kPaged4, SPLIT, false>(p, grid, stream);
  } else {
    launch_attn_v<BLK, kPagedAny, SPLIT, false>(p, grid, stream);
  }
}

}  // namespace

int attn_rows_per_wg() { return kRowsPerWG; }

hipError_t launch_attn(const AttnParams& p, hipStream_t stream) {
  const int64_t n_pool8 = p.kbar16 ? (int64_t)p.Hkv * p.kpitch * kHeadDim / 8 : 0;
  const int64_t n_kv8 = p.fp8 ? p.kv_elems / 8 : 0;
  if (n_pool8 + n_kv8 > 0) {
    const int64_t work = 2 * n_pool8 + n_kv8;
    const int blocks = (int)(work < 8192 * 256 ? (work + 255) / 256 : 8192);
    hipLaunchKernelGGL(prep_kernel, dim3(blocks), dim3(256), 0, stream, p, n_pool8, n_kv8);
  }
  const int64_t wgs = (int64_t)p.Hkv * p.NBq_tot * p.subs * p.splits;
  dim3 grid((unsigned)wgs);
  if (p.splits > 1) {
    if (p.B == 128) launch_attn_t<128, true>(p, grid, stream);
    else launch_attn_t<64, true>(p, grid, stream);
  } else {
    if (p.B == 128) launch_attn_t<128, false>(p, grid, stream);
    else launch_attn_t<64, false>(p, grid, stream);
  }
  if (p.splits > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)p.T * p.Hq;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((rows + 7) / 8)), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace fpv2
