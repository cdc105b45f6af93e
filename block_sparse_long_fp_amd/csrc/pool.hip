// Stage 1a: block-mean pooling of GQA-packed Q, and of K and V.
//
// Method: "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context LLM
// Serving" (metallab.ai paper digest), Figure 3 (Stage 1 packs the grouped
// queries and pools block-mean statistics) and Figure 4 (a pruned block is
// represented by its mean key and mean value).
//
// Work split: one workgroup per (key block b of the ragged batch, KV head h),
// the heads of one block consecutive. Its
// threads own "slots" (the G query heads of the group, then K, then V) times
// 16-byte column chunks of the 128-wide head dim, and split the block's tokens
// into interleaved groups; every load is a 16-byte (bf16) or 8-byte (fp8)
// vector whose neighbours in the wave read the neighbouring bytes of the same
// row, so each wave streams whole 128-byte lines. Partial sums meet in LDS in
// a fixed order (deterministic), are divided by the element count and written
// as fp32. The kernel is HBM-bound: it reads every input byte once.
//
// In chunked prefill a request's queries are its last positions; key blocks
// before the chunk (J < qb0) pool K and V only, and key block J >= qb0 also
// pools query block J - qb0 (the same positions, so the same token count).
// The chunk-only variant (fp_pool_chunk_blocks) runs one workgroup per query
// block and so pools only the key blocks J >= qb0 the chunk adds.
#include "common.h"
#include "launch.h"

namespace fpv2 {

namespace {

// Threads per workgroup: 256 when the grid has enough workgroups to keep
// every CU streaming; 1024 for small grids (pooling one short chunk), where a
// thread would otherwise sum its share of the block's tokens in many serial
// rounds of loads.
constexpr int kPoolThreadsWide = 1024;
constexpr int kPoolSmallGrid = 2048;
// A block's tokens are split into interleaved groups, each summed by one
// (group, slot, chunk) task in a fixed order and the partial sums reduced in
// a fixed order: about kPairs tasks per workgroup, whatever its thread count,
// so the pooled values do not depend on the launch shape (a chunk pooled
// alone equals the same block pooled with the whole prompt, bit for bit).
constexpr int kPairs = 768;
constexpr int kChunks = kHeadDim / 8;  // 8 elements per chunk

// Loads in flight per thread: a thread of a 256-thread workgroup sums 16
// tokens of a 128-token block, all requested at once for contiguous bf16
// inputs (2 % faster at Llama 128K than two rounds of 8). Rounds of 8 stay
// for the wide workgroups of small grids (16 measured 4 % slower on a
// 2048-token chunk), for paged K / V, whose per-token page lookups then need
// more registers (16: 10 % slower on the varlen paged batch), and for FP8
// codes (level).
template <int kPoolThreads, bool PAGED, bool FP8>
constexpr int kBatch = kPoolThreads == 256 && !PAGED && !FP8 ? 16 : 8;

// The 8 elements at `elem` as raw words (16 bytes of bf16, or 8 bytes of
// FP8 codes in .x/.y). Non-temporal loads: every input byte is read once, so
// the lines need not stay in L2 or MALL (Llama 128K: 0.295 -> 0.265 ms).
template <bool FP8>
__device__ __forceinline__ uint4 load_raw(const void* base, int64_t elem) {
  if constexpr (FP8) {
    const u32x2 w =
        __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(base) + elem));
    return make_uint4(w.x, w.y, 0, 0);
  } else {
    const u32x4 w =
        __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem));
    return make_uint4(w.x, w.y, w.z, w.w);
  }
}

// FP8 codes are widened with the gfx950 conversion v_cvt_scalef32_pk_f32_fp8
// (two codes per instruction, scale 1: exact, every E4M3 value is an fp32
// value), which keeps the FP8 pass bound by memory rather than by decoding.
template <bool FP8>
__device__ __forceinline__ void add_raw(const uint4 w, float (&acc)[8]) {
  if constexpr (FP8) {
    const f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.x, 1.0f, false);
    const f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.x, 1.0f, true);
    const f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.y, 1.0f, false);
    const f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.y, 1.0f, true);
    acc[0] += f0[0]; acc[1] += f0[1];
    acc[2] += f1[0]; acc[3] += f1[1];
    acc[4] += f2[0]; acc[5] += f2[1];
    acc[6] += f3[0]; acc[7] += f3[1];
  } else {
    acc[0] += bf16_lo(w.x); acc[1] += bf16_hi(w.x);
    acc[2] += bf16_lo(w.y); acc[3] += bf16_hi(w.y);
    acc[4] += bf16_lo(w.z); acc[5] += bf16_hi(w.z);
    acc[6] += bf16_lo(w.w); acc[7] += bf16_hi(w.w);
  }
}

// acc += the chunks at elem0 + k * estride for k = 0 .. cnt-1, in that order,
// NB loads in flight (the last batch's loads predicated).
template <bool FP8, int NB>
__device__ __forceinline__ void sum_strided(const void* base, int64_t elem0, int64_t estride, int cnt,
                                            float (&acc)[8]) {
  for (int k = 0; k < cnt; k += NB) {
    uint4 w[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u)
      w[u] = k + u < cnt ? load_raw<FP8>(base, elem0 + (int64_t)(k + u) * estride) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (k + u < cnt) add_raw<FP8>(w[u], acc);
  }
}

template <bool FP8, int kPoolThreads, bool PAGED>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(PoolParams p) {
  extern __shared__ float part[];  // [groups][slots*kChunks][8]
  // Consecutive workgroups are the KV heads of one block, so the workgroups
  // running together read whole token rows of Q, K and V.
  const int h = (int)(blockIdx.x % (unsigned)p.Hkv);
  const int bid = (int)(blockIdx.x / (unsigned)p.Hkv);
  const ReqTable& rt = p.rt;
  // bid: a global key block id in [0, NBk_tot), or with chunk_only a global
  // query block id in [0, NBq_tot) whose key block is pooled.
  int r = 0;
  int J;
  if (p.chunk_only) {
    while (r + 1 < rt.R && rt.blk_off[r + 1] <= bid) ++r;
    J = rt.qb0[r] + bid - rt.blk_off[r];
  } else {
    while (r + 1 < rt.R && rt.kblk_off[r + 1] <= bid) ++r;
    J = bid - rt.kblk_off[r];
  }
  const int b = rt.prow_off[r] + J;  // k_bar / v_bar row of key block J (per KV head)
  const int L = rt.ktok_off[r + 1] - rt.ktok_off[r];
  const int t0 = J * p.B;
  const int n = min(p.B, L - t0);
  const int qi = J - rt.qb0[r];    // query block of the call at these positions
  const bool has_q = qi >= 0;
  const int64_t qtok0 = (int64_t)rt.tok_off[r] + (int64_t)qi * p.B;

  if (p.sel_ticket != nullptr && blockIdx.x == 0) {
    // fp_stage1: clear the selection kernel's ticket and look-back states
    // (the selection launch that follows on the stream reads them).
    if (threadIdx.x == 0) *p.sel_ticket = 0u;
    for (int j = threadIdx.x; j < p.sel_words; j += kPoolThreads) p.sel_status[j] = 0ull;
  }

  constexpr int NB = kBatch<kPoolThreads, PAGED, FP8>;
  const int G = p.G;
  const int slots = G + 2;
  const int tasks = slots * kChunks;
  const int groups = tasks >= kPairs ? 1 : kPairs / tasks;
  const int tid = threadIdx.x;

  for (int tk = tid; tk < groups * tasks; tk += kPoolThreads) {
    const int task = tk % tasks;
    const int grp = tk / tasks;
    const int slot = task / kChunks;
    const int chunk = task % kChunks;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // This thread's tokens: grp, grp + groups, ... below n.
    const int cnt = grp < n ? (n - grp + groups - 1) / groups : 0;
    if (slot < G) {
      const int g = h * G + slot;
      if (has_q)
        sum_strided<FP8, NB>(p.q, ((qtok0 + grp) * p.Hq + g) * kHeadDim + chunk * 8,
                             (int64_t)groups * p.Hq * kHeadDim, cnt, acc);
    } else {
      const void* src = (slot == G) ? p.k : p.v;
      if constexpr (!PAGED) {
        sum_strided<FP8, NB>(src, kv_elem_offset(p.kv, rt, r, t0 + grp, h, p.Hkv) + chunk * 8,
                             (int64_t)groups * p.Hkv * kHeadDim, cnt, acc);
      } else {
        // Paged: a batch's page-table lookups go out together, then its loads
        // (the last batch predicated).
        for (int k = 0; k < cnt; k += NB) {
          int64_t off[NB];
#pragma unroll
          for (int u = 0; u < NB; ++u)
            off[u] = k + u < cnt ? kv_elem_offset(p.kv, rt, r, t0 + grp + (k + u) * groups, h, p.Hkv) + chunk * 8
                                 : 0;
          uint4 w[NB];
#pragma unroll
          for (int u = 0; u < NB; ++u) w[u] = k + u < cnt ? load_raw<FP8>(src, off[u]) : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int u = 0; u < NB; ++u)
            if (k + u < cnt) add_raw<FP8>(w[u], acc);
        }
      }
    }
    float* dst = part + ((int64_t)grp * tasks + task) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = acc[i];
  }
  __syncthreads();

  // Reduce: one thread per (output kind, chunk): kind 0 = q_bar, 1 = k_bar, 2 = v_bar.
  if (tid < 3 * kChunks && (has_q || tid >= kChunks)) {
    const int kind = tid / kChunks;
    const int c = tid % kChunks;
    float s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = 0.f;
    const int s_lo = (kind == 0) ? 0 : (kind == 1 ? G : G + 1);
    const int s_hi = (kind == 0) ? G : s_lo + 1;
    for (int sl = s_lo; sl < s_hi; ++sl) {
      for (int gr = 0; gr < groups; ++gr) {
        const float* src = part + ((int64_t)gr * tasks + sl * kChunks + c) * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] += src[i];
      }
    }
    float scale;
    if (kind == 0) {
      scale = 1.0f / (float)(n * G);
      if (FP8) scale *= *p.descale_q;
    } else {
      scale = 1.0f / (float)n;
      if (FP8) scale *= (kind == 1) ? *p.descale_k : *p.descale_v;
    }
    float* out = (kind == 0) ? p.q_bar : (kind == 1 ? p.k_bar : p.v_bar);
    const int64_t orow = kind == 0 ? (int64_t)h * p.NBq_tot + rt.blk_off[r] + qi : (int64_t)h * p.kpitch + b;
    float4* o4 = reinterpret_cast<float4*>(out + orow * kHeadDim + c * 8);
    o4[0] = make_float4(s[0] * scale, s[1] * scale, s[2] * scale, s[3] * scale);
    o4[1] = make_float4(s[4] * scale, s[5] * scale, s[6] * scale, s[7] * scale);
  }
}

}  // namespace

size_t pool_lds_bytes(int G) {
  const int tasks = (G + 2) * kChunks;
  const int groups = tasks >= kPairs ? 1 : kPairs / tasks;
  return (size_t)groups * tasks * 8 * sizeof(float);
}

template <bool FP8, int kThreads>
static void launch_pool_as(const PoolParams& p, unsigned wgs, size_t lds, hipStream_t stream) {
  if (p.kv.paged)
    hipLaunchKernelGGL((pool_kernel<FP8, kThreads, true>), dim3(wgs), dim3(kThreads), lds, stream, p);
  else
    hipLaunchKernelGGL((pool_kernel<FP8, kThreads, false>), dim3(wgs), dim3(kThreads), lds, stream, p);
}

hipError_t launch_pool(const PoolParams& p, hipStream_t stream) {
  const unsigned wgs = (unsigned)p.Hkv * (unsigned)(p.chunk_only ? p.NBq_tot : p.NBk_tot);
  const size_t lds = pool_lds_bytes(p.G);
  if (wgs >= (unsigned)kPoolSmallGrid) {
    if (p.fp8) launch_pool_as<true, 256>(p, wgs, lds, stream);
    else launch_pool_as<false, 256>(p, wgs, lds, stream);
  } else {
    if (p.fp8) launch_pool_as<true, kPoolThreadsWide>(p, wgs, lds, stream);
    else launch_pool_as<false, kPoolThreadsWide>(p, wgs, lds, stream);
  }
  return hipGetLastError();
}

}  // namespace fpv2
