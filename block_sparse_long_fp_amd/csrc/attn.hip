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
//     O^T = V^T P^T with v_mfma_f32_32x32x16_bf16. A lane (column c, half hf)
//     holds the scores and output dims of query c, so row max and row sum are
//     in-lane plus one exchange with lane c+32, and the probabilities feed the
//     PV product straight from registers (the PV contraction index is
//     relabelled to match the score accumulator layout; V^T is read from LDS
//     with the same relabelling).
//   * Work items: the CSR row's key blocks (B keys), then correction chunks of
//     64 pooled columns whose per-column bias log2(n_J) or -inf masks selected
//     and non-causal blocks (from an LDS bitmap of the row). Every item
//     reaches LDS as bf16 K rows and bf16 V^T columns, so the MFMA code has
//     one path.
//   * Staging: the next item's K and V pass through 32 registers per thread
//     (loaded before the current item is computed, stored after it) into
//     double-buffered LDS, with one workgroup barrier per item. K is
//     row-major with a 272-byte pitch, V^T has a (B+4)-element pitch: MFMA
//     operand reads of consecutive rows are bank-conflict free and use
//     base + immediate addresses. Stores are mapped key-group-fastest so each
//     32-lane pass writes one contiguous row segment (no conflicts).
//   * Wave-uniform quantities live in scalar registers, so per-item and
//     per-tile decisions are scalar branches.
//   * Online softmax in base 2, updated per 64-key half of an item (32 score
//     registers live, which keeps the kernel within 256 VGPRs without
//     spills): max on raw scores, one fma + exp2 per score, fp32 row sums. The running max only moves when a block's max exceeds it
//     by more than 8 (probabilities stay below 256, exact after the final
//     division), which makes output rescales rare.
//   * Workgroups run heaviest first (query block index descending over the
//     ragged batch), and consecutive ids cycle over KV heads so the
//     round-robin XCD dispatch keeps one KV head's blocks in one XCD's L2.
#include "common.h"
#include "launch.h"

namespace fpv2 {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWG = kWaves * 32;
constexpr int kPC = 64;                 // pooled columns per correction item
constexpr int kKPitch = kHeadDim + 8;   // bf16 elements per K row in LDS (272 B)
constexpr int kColCache = 1024;         // CSR columns cached in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;
constexpr float kSlack = 8.0f;          // lazy-rescale threshold of the running max (log2)

template <int BLK>
struct Lds {
  static constexpr int kVPitch = BLK + 4;  // bf16 elements per V^T row
  uint16_t k[2][BLK * kKPitch];
  uint16_t vt[2][kHeadDim * kVPitch];
  float bias[2][kPC];
  uint32_t selbits[FP_MAX_BLOCKS_PER_SEQ / 32];
  int32_t colcache[kColCache];
};

// Load 8 consecutive elements (bf16 or fp8) as 8 bf16 in a uint4.
template <bool FP8>
__device__ __forceinline__ uint4 load8_as_bf16(const void* base, int64_t elem) {
  if constexpr (FP8) {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(base) + elem);
    uint4 o;
    o.x = pack_bf16x2(e4m3_to_float(w.x & 0xFF), e4m3_to_float((w.x >> 8) & 0xFF));
    o.y = pack_bf16x2(e4m3_to_float((w.x >> 16) & 0xFF), e4m3_to_float(w.x >> 24));
    o.z = pack_bf16x2(e4m3_to_float(w.y & 0xFF), e4m3_to_float((w.y >> 8) & 0xFF));
    o.w = pack_bf16x2(e4m3_to_float((w.y >> 16) & 0xFF), e4m3_to_float(w.y >> 24));
    return o;
  } else {
    return *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem);
  }
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Per-workgroup constants of the row being processed (all wave-uniform).
struct RowCtx {
  int r, I, h, L;
  int n_exact;          // CSR entries (key blocks) of the row
  int n_items;          // plus the correction chunks
  const int32_t* cols;  // CSR row (nullptr in dense mode)
  int64_t pooled_base;  // element offset of the k_bar/v_bar row (h, blk_off[r])
  int64_t tok_base;     // first token of the request
  float kscale;         // pooled k_bar -> LDS scale (1/descale_k for FP8)
  float vscale;         // pooled v_bar -> LDS scale (1/descale_v for FP8)
};

// Element offset of key `row` of block J (request-local token J*B+row, clamped
// to the request's last token) of the row's KV head.
template <int BLK, bool PAGED>
__device__ __forceinline__ int64_t kv_off(const AttnParams& p, const RowCtx& rc, int J, int row) {
  const int rr = min(row, rc.L - 1 - J * BLK);
  if constexpr (!PAGED) {
    const int64_t base = ((rc.tok_base + (int64_t)J * BLK) * p.Hkv + rc.h) * kHeadDim;
    return base + (int64_t)(rr * (p.Hkv * kHeadDim));
  } else {
    const int t = J * BLK + rr;
    const int page = p.kv.page_table[(int64_t)rc.r * p.kv.max_pages + t / p.kv.page_size];
    return (((int64_t)page * p.kv.page_size + (t % p.kv.page_size)) * p.Hkv + rc.h) * kHeadDim;
  }
}

// Staging of one item from HBM to LDS: every thread issues the same eight
// 16-byte loads (stage slots) from one straight-line sequence whatever the
// item kind (only the addresses are chosen per kind), so the loads stay in
// flight while the current item is computed and no register copies merge
// them afterwards. Slot plans, with E = elements per 16 bytes (8 bf16 or
// 16 fp8) and C = d / E loads per key row:
//   exact K: slot u < KL holds row tid/C + (512/C)u, elements E(tid%C)..;
//            KL = B*C/512 (bf16: 4 at B=128, 2 at B=64; fp8: 2 or 1).
//   exact V: slot 4+i (i < KL) holds key KL*kg + i (kg = tid % (B/KL)),
//            elements E(tid / (B/KL)).., so each thread owns KL consecutive
//            keys of E dims and writes V^T rows directly.
//   Unused exact slots repeat a used address (the load hits the same line).
//   pooled K: slots 2u, 2u+1 hold fp32 row tid/16 + 32u (u < 2), dims 8(tid%16)..
//   pooled V: slots 4+2i, 5+2i hold fp32 column 2kg+i (kg = tid%32), dims 8(tid/32)..
struct Stage {
  uint4 x[8];
};

template <int BLK, bool FP8>
struct ExactPlan {
  static constexpr int E = FP8 ? 16 : 8;
  static constexpr int C = kHeadDim / E;
  static constexpr int KL = BLK * C / kThreads;
  static constexpr int KG = BLK / KL;
  static_assert(KL >= 1 && KL <= 4 && KG * C == kThreads, "exact staging plan");
};

template <int BLK, bool FP8, bool PAGED>
__device__ __forceinline__ void load_item(Stage& st, const AttnParams& p, const RowCtx& rc, const int32_t* colcache,
                                          int e, int tid) {
  using P = ExactPlan<BLK, FP8>;
  g_u32x4* src[8];  // global address space, so the loads stay global (not flat)
  if (e < rc.n_exact) {
    const int J = !rc.cols ? e : uniform(e < kColCache ? lload_i32(colcache + e) : gload_i32(rc.cols + e));
    g_uint8* kbase = (g_uint8*)p.k;
    g_uint8* vbase = (g_uint8*)p.v;
    constexpr int eb = FP8 ? 1 : 2;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int uu = u % P::KL;
      const int64_t off = kv_off<BLK, PAGED>(p, rc, J, tid / P::C + (kThreads / P::C) * uu) + (tid % P::C) * P::E;
      src[u] = (g_u32x4*)(kbase + off * eb);
    }
    const int kg = tid % P::KG, dc = tid / P::KG;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ii = i % P::KL;
      const int64_t off = kv_off<BLK, PAGED>(p, rc, J, kg * P::KL + ii) + dc * P::E;
      src[4 + i] = (g_u32x4*)(vbase + off * eb);
    }
  } else {
    const int c0 = (e - rc.n_exact) * kPC;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int Jp = min(c0 + (tid >> 4) + 32 * u, rc.I - 1);
      g_u32x4* s = (g_u32x4*)((g_float*)p.k_bar + rc.pooled_base + (int64_t)Jp * kHeadDim + (tid & 15) * 8);
      src[2 * u] = s;
      src[2 * u + 1] = s + 1;
    }
    const int kg = tid & 31, dc = tid >> 5;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int Jp = min(c0 + kg * 2 + i, rc.I - 1);
      g_u32x4* s = (g_u32x4*)((g_float*)p.v_bar + rc.pooled_base + (int64_t)Jp * kHeadDim + dc * 8);
      src[4 + 2 * i] = s;
      src[5 + 2 * i] = s + 1;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) st.x[i] = gload16(src[i]);
}

__device__ __forceinline__ uint4 cvt8(const uint4 a4, const uint4 b4, float s) {
  const float4 a = __builtin_bit_cast(float4, a4), b = __builtin_bit_cast(float4, b4);
  uint4 o;
  o.x = pack_bf16x2(a.x * s, a.y * s);
  o.y = pack_bf16x2(a.z * s, a.w * s);
  o.z = pack_bf16x2(b.x * s, b.y * s);
  o.w = pack_bf16x2(b.z * s, b.w * s);
  return o;
}

// The 16 e4m3 codes of a slot as 16 floats (exact).
__device__ __forceinline__ void fp8x16_to_float(const uint4 w, float (&f)[16]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int b = 0; b < 4; ++b) f[4 * q + b] = e4m3_to_float((ws[q] >> (8 * b)) & 0xFFu);
}

template <int BLK, bool FP8>
__device__ __forceinline__ void store_item(const Stage& st, Lds<BLK>& sm, int buf, const RowCtx& rc, int e, int tid) {
  using P = ExactPlan<BLK, FP8>;
  constexpr int VP = Lds<BLK>::kVPitch;
  uint16_t* kb = sm.k[buf];
  uint16_t* vt = sm.vt[buf];
  if (e < rc.n_exact) {
#pragma unroll
    for (int u = 0; u < P::KL; ++u) {
      uint16_t* d = &kb[(tid / P::C + (kThreads / P::C) * u) * kKPitch + (tid % P::C) * P::E];
      if constexpr (!FP8) {
        *reinterpret_cast<uint4*>(d) = st.x[u];
      } else {
        float f[16];
        fp8x16_to_float(st.x[u], f);
        uint4 lo, hi;
        lo.x = pack_bf16x2(f[0], f[1]);
        lo.y = pack_bf16x2(f[2], f[3]);
        lo.z = pack_bf16x2(f[4], f[5]);
        lo.w = pack_bf16x2(f[6], f[7]);
        hi.x = pack_bf16x2(f[8], f[9]);
        hi.y = pack_bf16x2(f[10], f[11]);
        hi.z = pack_bf16x2(f[12], f[13]);
        hi.w = pack_bf16x2(f[14], f[15]);
        reinterpret_cast<uint4*>(d)[0] = lo;
        reinterpret_cast<uint4*>(d)[1] = hi;
      }
    }
    const int kg = tid % P::KG, dc = tid / P::KG;
    uint16_t* d = vt + (dc * P::E) * VP + kg * P::KL;
    if constexpr (!FP8 && P::KL == 4) {
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&st.x[4]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&st.x[5]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&st.x[6]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&st.x[7]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint2 lo, hi;
        lo.x = __builtin_amdgcn_perm(w1[m], w0[m], 0x05040100u);  // keys 0,1 of dim 2m
        lo.y = __builtin_amdgcn_perm(w3[m], w2[m], 0x05040100u);  // keys 2,3 of dim 2m
        hi.x = __builtin_amdgcn_perm(w1[m], w0[m], 0x07060302u);  // dim 2m+1
        hi.y = __builtin_amdgcn_perm(w3[m], w2[m], 0x07060302u);
        *reinterpret_cast<uint2*>(d + (2 * m) * VP) = lo;
        *reinterpret_cast<uint2*>(d + (2 * m + 1) * VP) = hi;
      }
    } else if constexpr (!FP8 && P::KL == 2) {
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&st.x[4]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&st.x[5]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        *reinterpret_cast<uint32_t*>(d + (2 * m) * VP) = __builtin_amdgcn_perm(w1[m], w0[m], 0x05040100u);
        *reinterpret_cast<uint32_t*>(d + (2 * m + 1) * VP) = __builtin_amdgcn_perm(w1[m], w0[m], 0x07060302u);
      }
    } else if constexpr (FP8 && P::KL == 2) {
      float f0[16], f1[16];
      fp8x16_to_float(st.x[4], f0);
      fp8x16_to_float(st.x[5], f1);
#pragma unroll
      for (int q = 0; q < 16; ++q) *reinterpret_cast<uint32_t*>(d + q * VP) = pack_bf16x2(f0[q], f1[q]);
    } else {
      static_assert(FP8 && P::KL == 1, "exact V staging plan");
      float f0[16];
      fp8x16_to_float(st.x[4], f0);
#pragma unroll
      for (int q = 0; q < 16; ++q) d[q * VP] = static_cast<uint16_t>(pack_bf16x2(f0[q], 0.f));
    }
  } else {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      *reinterpret_cast<uint4*>(&kb[((tid >> 4) + 32 * u) * kKPitch + (tid & 15) * 8]) =
          cvt8(st.x[2 * u], st.x[2 * u + 1], rc.kscale);
    const int kg = tid & 31, dc = tid >> 5;
    uint16_t* d = vt + (dc * 8) * VP + kg * 2;
    const float4 a0 = __builtin_bit_cast(float4, st.x[4]), a1 = __builtin_bit_cast(float4, st.x[5]);
    const float4 b0 = __builtin_bit_cast(float4, st.x[6]), b1 = __builtin_bit_cast(float4, st.x[7]);
    const float x0[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float x1[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    const float s = rc.vscale;
#pragma unroll
    for (int q = 0; q < 8; ++q) *reinterpret_cast<uint32_t*>(d + q * VP) = pack_bf16x2(x0[q] * s, x1[q] * s);
    if (tid < kPC) {
      const int Jc = (e - rc.n_exact) * kPC + tid;
      float bv = -INFINITY;
      if (Jc < rc.I && !((sm.selbits[Jc >> 5] >> (Jc & 31)) & 1u)) bv = __log2f((float)min(BLK, rc.L - Jc * BLK));
      sm.bias[buf][tid] = bv;
    }
  }
}

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
  static constexpr int NKT = BLK / 32;
  bf16x8 qf[kHeadDim / 16];  // B operand of S^T = K Q^T, one per 16-dim step
  f32x16 o[kHeadDim / 32];   // O^T accumulators, one per 32-dim tile
  float m;                   // running max (log2 units)
  float l;                   // this lane's partial row sum
};

// Item kinds: a selected key block off the diagonal (all keys visible), the
// diagonal block (causal mask inside tile kt_lim), or a chunk of pooled
// columns (logit s*sl2 + bias[col]; columns past the chunk end have bias
// -inf). Each kind is its own instantiation so the common case carries no
// per-score masking or bias work.
enum ItemKind { kExact = 0, kDiag = 1, kPooled = 2 };

// One item for one wave, processed in 64-key halves (each: QK^T of two
// 32-key tiles, online-softmax update, PV), which keeps 32 score registers
// live instead of 64. kt_lim: last 32-key tile that is not fully masked.
template <int BLK, int KIND>
__device__ __forceinline__ void attend_item(WaveState<BLK>& ws, const uint16_t* kb, const uint16_t* vt,
                                            const float* bias, int kt_lim_rt, int tq, float sl2, int lk, int lv,
                                            int hf) {
  constexpr int NKT = BLK / 32;
  constexpr int VP = Lds<BLK>::kVPitch;
  const int kt_lim = KIND == kExact ? NKT - 1 : kt_lim_rt;
#pragma unroll
  for (int hh = 0; hh < NKT / 2; ++hh) {
    if (KIND != kExact && 2 * hh > kt_lim) break;
    // Tile 2hh+1 of a half is skipped when it lies past kt_lim (diagonal or
    // short pooled chunk); its scores are then never read.
    const bool two = KIND == kExact || 2 * hh + 1 <= kt_lim;
    f32x16 s[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int kt = 2 * hh + t2;
      if (t2 == 1 && !two) {
        s[1] = f32x16{};
        continue;
      }
      const uint16_t* base = kb + lk + kt * 32 * kKPitch;
      f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(base), ws.qf[0],
                                                           f32x16{}, 0, 0, 0);
#pragma unroll
      for (int ks = 1; ks < kHeadDim / 16; ++ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(base + ks * 16),
                                                      ws.qf[ks], acc, 0, 0, 0);
      s[t2] = acc;
    }
    float mx;
    if constexpr (KIND == kPooled) {
      mx = kNegBig;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int kt = 2 * hh + t2;
        if (t2 == 1 && !two) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 bb = *reinterpret_cast<const float4*>(&bias[kt * 32 + i * 8 + hf * 4]);
          const float bv[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            s[t2][4 * i + jj] = fmaf(s[t2][4 * i + jj], sl2, bv[jj]);
            mx = fmaxf(mx, s[t2][4 * i + jj]);
          }
        }
      }
    } else {
      if constexpr (KIND == kDiag) {
        // Mask keys past the query in tile kt_lim (the only partial tile).
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const int kt = 2 * hh + t2;
          if (kt == kt_lim) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int jj = 0; jj < 4; ++jj)
                if (kt * 32 + i * 8 + hf * 4 + jj > tq) s[t2][4 * i + jj] = -INFINITY;
          }
        }
      }
      mx = kNegBig;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        if (t2 == 1 && !two) break;
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[t2][e]);
      }
      mx *= sl2;
    }
    mx = max_halves(mx);
    // Lazy running max (see the file header).
    const float m_new = mx > ws.m + kSlack ? mx : ws.m;
    if (__ballot(m_new != ws.m) != 0) {
      const float corr = __builtin_amdgcn_exp2f(ws.m - m_new);
      ws.l *= corr;
#pragma unroll
      for (int dt = 0; dt < kHeadDim / 32; ++dt) ws.o[dt] *= corr;
    }
    ws.m = m_new;
    const float sc = KIND == kPooled ? 1.0f : sl2;
    const float neg_m = -m_new;
    float lsum0 = 0.f;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int kt = 2 * hh + t2;
      if (t2 == 1 && !two) break;
      bf16x8 pf[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        float pv[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) pv[t] = __builtin_amdgcn_exp2f(fmaf(s[t2][8 * s2 + t], sc, neg_m));
#pragma unroll
        for (int t = 0; t < 8; ++t) lsum0 += pv[t];
        const bf16x4 lo = __builtin_convertvector(f32x4{pv[0], pv[1], pv[2], pv[3]}, bf16x4);
        const bf16x4 hi = __builtin_convertvector(f32x4{pv[4], pv[5], pv[6], pv[7]}, bf16x4);
        pf[s2] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int dt = 0; dt < kHeadDim / 32; ++dt) {
        const uint16_t* base = vt + lv + dt * 32 * VP + kt * 32;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const uint2 lo = *reinterpret_cast<const uint2*>(base + s2 * 16);
          const uint2 hi = *reinterpret_cast<const uint2*>(base + s2 * 16 + 8);
          const u32x4 wv = {lo.x, lo.y, hi.x, hi.y};
          ws.o[dt] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wv), pf[s2], ws.o[dt], 0, 0, 0);
        }
      }
    }
    ws.l += lsum0;
  }
}

// blockIdx -> (query block I, request r) in descending-I order over the ragged
// batch, plus (kv head, sub-tile).
__device__ __forceinline__ void decode_work(const AttnParams& p, int& I, int& r, int& h, int& sub) {
  const ReqTable& rt = p.rt;
  const int U = p.Hkv * p.subs;
  const int pk = blockIdx.x / U;
  const int rem = blockIdx.x - pk * U;
  h = rem % p.Hkv;
  sub = rem / p.Hkv;
  // C(x) = number of (r, I') with I' > x; non-increasing. Smallest I with C(I) <= pk.
  auto C = [&](int x) {
    int s = 0;
    for (int q = 0; q < rt.R; ++q) s += max(0, rt.blk_off[q + 1] - rt.blk_off[q] - 1 - x);
    return s;
  };
  int lo = 0, hi = rt.nb_max - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (C(mid) <= pk) hi = mid;
    else lo = mid + 1;
  }
  I = lo;
  int j = pk - C(I);
  r = 0;
  for (int q = 0; q < rt.R; ++q) {
    if (rt.blk_off[q + 1] - rt.blk_off[q] > I) {
      if (j == 0) { r = q; break; }
      --j;
    }
  }
}

template <int BLK, bool FP8, bool PAGED>
__global__ __launch_bounds__(kThreads, 1) void attn_kernel(AttnParams p) {
  __shared__ Lds<BLK> sm;
  constexpr int NKT = BLK / 32;
  RowCtx rc;
  int sub;
  decode_work(p, rc.I, rc.r, rc.h, sub);
  const ReqTable& rt = p.rt;
  rc.tok_base = rt.tok_off[rc.r];
  rc.L = rt.tok_off[rc.r + 1] - rt.tok_off[rc.r];
  const int I = rc.I;
  const int nI = min(BLK, rc.L - I * BLK);
  const int64_t row = (int64_t)rc.h * p.NB_tot + rt.blk_off[rc.r] + I;
  rc.n_exact = p.dense ? I + 1 : p.row_ptr[row + 1] - p.row_ptr[row];
  rc.cols = p.dense ? nullptr : p.col_idx + p.row_ptr[row];
  const bool do_corr = p.mean_correction && !p.dense && I > 0;
  rc.n_items = rc.n_exact + (do_corr ? (I + kPC - 1) / kPC : 0);
  rc.pooled_base = ((int64_t)rc.h * p.NB_tot + rt.blk_off[rc.r]) * kHeadDim;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int c = lane & 31, hf = lane >> 5;
  const int prow0 = sub * kRowsPerWG + w * 32;  // first packed row of this wave
  const bool wave_active = prow0 < p.G * BLK;
  const int g = rc.h * p.G + (wave_active ? prow0 / BLK : 0);
  const int tq0 = prow0 % BLK;
  const int tq = tq0 + c;
  const bool q_valid = wave_active && tq < nI;
  const int64_t tok = rc.tok_base + (int64_t)I * BLK + tq;
  const int lk = c * kKPitch + hf * 8;              // K operand base of this lane
  const int lv = c * Lds<BLK>::kVPitch + hf * 4;    // V^T operand base of this lane

  // Logit scale in log2 units; FP8 folds both descales into it and stages
  // pooled k_bar / v_bar divided by the K / V descales (so both streams stay
  // in code units), and multiplies the output by the V descale.
  float sl2 = p.sm_scale * kLog2e;
  rc.kscale = 1.f;
  rc.vscale = 1.f;
  float oscale = 1.f;
  if constexpr (FP8) {
    const float dq = *p.descale_q, dk = *p.descale_k, dv = *p.descale_v;
    sl2 *= dq * dk;
    rc.kscale = 1.f / dk;
    rc.vscale = 1.f / dv;
    oscale = dv;
  }

  WaveState<BLK> ws;
  ws.m = kNegBig;
  ws.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < kHeadDim / 32; ++dt) ws.o[dt] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < kHeadDim / 16; ++ks) {
    uint4 qv = make_uint4(0, 0, 0, 0);
    if (q_valid) qv = load8_as_bf16<FP8>(p.q, (tok * p.Hq + g) * kHeadDim + ks * 16 + hf * 8);
    ws.qf[ks] = __builtin_bit_cast(bf16x8, qv);
  }

  if (!p.dense) {
    if (do_corr)
      for (int wd = tid; wd <= (I >> 5); wd += kThreads) sm.selbits[wd] = 0u;
    for (int e = tid; e < min(rc.n_exact, kColCache); e += kThreads) sm.colcache[e] = rc.cols[e];
    __syncthreads();
    if (do_corr) {
      for (int e = tid; e < rc.n_exact; e += kThreads) {
        const int J = e < kColCache ? lload_i32(sm.colcache + e) : gload_i32(rc.cols + e);
        atomicOr(&sm.selbits[J >> 5], 1u << (J & 31));
      }
    }
    __syncthreads();
  }

  const int N = rc.n_items;
  Stage st;
  load_item<BLK, FP8, PAGED>(st, p, rc, sm.colcache, 0, tid);
  store_item<BLK, FP8>(st, sm, 0, rc, 0, tid);
  __syncthreads();
  for (int e = 0; e < N; ++e) {
    const int buf = e & 1;
    // The thread index is laundered per item so the per-slot address terms
    // are recomputed (a few integer ops) instead of being held in registers
    // across the whole loop.
    int tid_l = tid;
    asm volatile("" : "+v"(tid_l));
    if (e + 1 < N) load_item<BLK, FP8, PAGED>(st, p, rc, sm.colcache, e + 1, tid_l);
    if (wave_active) {
      if (e < rc.n_exact - 1)
        attend_item<BLK, kExact>(ws, sm.k[buf], sm.vt[buf], sm.bias[buf], NKT - 1, tq, sl2, lk, lv, hf);
      else if (e == rc.n_exact - 1)
        attend_item<BLK, kDiag>(ws, sm.k[buf], sm.vt[buf], sm.bias[buf], tq0 >> 5, tq, sl2, lk, lv, hf);
      else
        attend_item<BLK, kPooled>(ws, sm.k[buf], sm.vt[buf], sm.bias[buf],
                                  (min(kPC, I - (e - rc.n_exact) * kPC) - 1) >> 5, tq, sl2, lk, lv, hf);
    }
    int tid_s = tid;
    asm volatile("" : "+v"(tid_s));
    if (e + 1 < N) store_item<BLK, FP8>(st, sm, buf ^ 1, rc, e + 1, tid_s);
    __syncthreads();
  }

  if (!wave_active) return;
  const float l_tot = sum_halves(ws.l);
  if (q_valid) {
    const float inv = oscale / l_tot;
    uint16_t* orow = p.out + (tok * p.Hq + g) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < kHeadDim / 32; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 pk;
        pk.x = pack_bf16x2(ws.o[dt][4 * i + 0] * inv, ws.o[dt][4 * i + 1] * inv);
        pk.y = pack_bf16x2(ws.o[dt][4 * i + 2] * inv, ws.o[dt][4 * i + 3] * inv);
        *reinterpret_cast<uint2*>(orow + dt * 32 + i * 8 + hf * 4) = pk;
      }
    }
    if (p.lse != nullptr && hf == 0) p.lse[(int64_t)g * p.T + tok] = (ws.m + __log2f(l_tot)) * kLn2;
  }
}

template <int BLK, bool FP8>
void launch_attn_t(const AttnParams& p, dim3 grid, hipStream_t stream) {
  if (p.kv.paged) hipLaunchKernelGGL((attn_kernel<BLK, FP8, true>), grid, dim3(kThreads), 0, stream, p);
  else hipLaunchKernelGGL((attn_kernel<BLK, FP8, false>), grid, dim3(kThreads), 0, stream, p);
}

}  // namespace

int attn_rows_per_wg() { return kRowsPerWG; }

hipError_t launch_attn(const AttnParams& p, hipStream_t stream) {
  const int64_t wgs = (int64_t)p.Hkv * p.NB_tot * p.subs;
  dim3 grid((unsigned)wgs);
  if (p.B == 128) {
    if (p.fp8) launch_attn_t<128, true>(p, grid, stream);
    else launch_attn_t<128, false>(p, grid, stream);
  } else {
    if (p.fp8) launch_attn_t<64, true>(p, grid, stream);
    else launch_attn_t<64, false>(p, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace fpv2
