// Stage 2: block-sparse causal prefill attention with the fused mean correction.
//
// Method: "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context LLM
// Serving" (metallab.ai paper digest):
//   Figure 3  Stage 2 computes exact attention over the CSR-selected blocks
//             while unselected blocks are compensated by the mean-correction
//             path; both streams merge inside one online softmax.
//   Figure 4  a pruned block J contributes |B_J| exp(s_J) (v_bar_J, 1): here
//             the logit sm * q_i . k_bar_J + ln n_J on value v_bar_J.
//   Fig. 1 / "What they did"  PackGQA: the G query heads of one KV head are
//             packed into one tile so each K/V tile is fetched once for them.
//
// gfx950 design (not a translation of the pages' Hopper kernel):
//   * One workgroup = 8 waves = 256 packed query rows of one (KV head h, query
//     block I): wave w owns 32 consecutive tokens of one query head. G*B rows
//     per (h, I) are split over ceil(G*B/256) workgroups.
//   * Transposed products keep every lane on one query: S^T = K Q^T and
//     O^T = V^T P^T with v_mfma_f32_32x32x16_bf16. A lane (column c, half hf)
//     then holds 64 scores and 64 output dims of query c, so the row max and
//     row sum are in-lane plus one exchange with lane c+32, and the softmax
//     probabilities feed the PV product straight from registers (the PV
//     contraction index is relabelled to match the score accumulator layout,
//     and V^T is read from LDS with the same relabelling).
//   * K is staged in LDS row-major [key][d] (pitch 136 elements); V is staged
//     transposed [d][key] (pitch B+4) so the PV operand is two 8-byte reads.
//     The next selected block's K/V is loaded into registers while the
//     current block computes.
//   * Online softmax in base 2 with the scale folded into one multiply; the
//     output rescale is skipped when no lane's running max moved.
//   * The correction path stages B pooled keys/values at a time (fp32 ->
//     bf16) and masks selected or non-causal columns through a per-column bias
//     (log2 n_J or -inf) built from an LDS bitmap of the row's CSR entries.
//   * Workgroups run heaviest first (query block index descending over the
//     ragged batch), and consecutive ids cycle over KV heads so that the
//     round-robin XCD dispatch keeps one KV head's blocks in one XCD's L2.
#include "common.h"
#include "launch.h"

namespace fpv2 {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWG = kWaves * 32;
constexpr int kKPitch = kHeadDim + 8;  // bf16 elements per K row in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;

template <int BLK>
struct Smem {
  static constexpr int kVPitch = BLK + 4;  // bf16 elements per V^T row
  uint16_t k[BLK * kKPitch];
  uint16_t vt[kHeadDim * kVPitch];
  float bias[BLK];
  uint32_t selbits[FP_MAX_BLOCKS_PER_SEQ / 32];
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

// Register-staged copy of one key block (K rows and V rows) on its way to LDS.
template <int BLK>
struct KVStage {
  static constexpr int kKChunks = BLK * (kHeadDim / 8) / kThreads;  // 16-byte chunks of K per thread
  static constexpr int kVTasks = (BLK / 4) * (kHeadDim / 8);        // 4 keys x 8 dims per task
  uint4 k[kKChunks];
  uint4 v[4];
};

template <int BLK, bool FP8>
__device__ __forceinline__ void kv_load(KVStage<BLK>& st, const AttnParams& p, int r, int J, int h, int L) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < KVStage<BLK>::kKChunks; ++u) {
    const int ci = tid + u * kThreads;
    const int kk = ci >> 4, dc = ci & 15;
    const int t = J * BLK + kk;
    if ((unsigned)t < (unsigned)L) st.k[u] = load8_as_bf16<FP8>(p.k, kv_elem_offset(p.kv, p.rt, r, t, h, p.Hkv) + dc * 8);
    else st.k[u] = make_uint4(0, 0, 0, 0);
  }
  if (tid < KVStage<BLK>::kVTasks) {
    const int dc = tid & 15, kg = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = J * BLK + kg * 4 + i;
      if ((unsigned)t < (unsigned)L) st.v[i] = load8_as_bf16<FP8>(p.v, kv_elem_offset(p.kv, p.rt, r, t, h, p.Hkv) + dc * 8);
      else st.v[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

// Write 4 keys x 8 dims (v[i] = 8 dims of key i) transposed into V^T.
template <int BLK>
__device__ __forceinline__ void vt_store4x8(Smem<BLK>& sm, int kg, int dc, const uint4 (&v)[4]) {
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&v[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&v[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&v[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&v[3]);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    // dims 8dc+2m (low halves) and 8dc+2m+1 (high halves)
    uint2 lo, hi;
    lo.x = __builtin_amdgcn_perm(w1[m], w0[m], 0x05040100u);  // (k0.lo, k1.lo)
    lo.y = __builtin_amdgcn_perm(w3[m], w2[m], 0x05040100u);  // (k2.lo, k3.lo)
    hi.x = __builtin_amdgcn_perm(w1[m], w0[m], 0x07060302u);  // (k0.hi, k1.hi)
    hi.y = __builtin_amdgcn_perm(w3[m], w2[m], 0x07060302u);
    *reinterpret_cast<uint2*>(&sm.vt[(dc * 8 + 2 * m) * Smem<BLK>::kVPitch + kg * 4]) = lo;
    *reinterpret_cast<uint2*>(&sm.vt[(dc * 8 + 2 * m + 1) * Smem<BLK>::kVPitch + kg * 4]) = hi;
  }
}

template <int BLK>
__device__ __forceinline__ void kv_store(const KVStage<BLK>& st, Smem<BLK>& sm) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < KVStage<BLK>::kKChunks; ++u) {
    const int ci = tid + u * kThreads;
    const int kk = ci >> 4, dc = ci & 15;
    *reinterpret_cast<uint4*>(&sm.k[kk * kKPitch + dc * 8]) = st.k[u];
  }
  if (tid < KVStage<BLK>::kVTasks) vt_store4x8<BLK>(sm, tid >> 4, tid & 15, st.v);
}

// Stage B pooled keys/values of correction chunk cb (fp32 -> bf16) plus the
// per-column bias: log2(n_J) for a pruned causal block, -inf otherwise.
// Returns (through LDS) nothing; the caller syncs.
template <int BLK>
__device__ __forceinline__ void stage_pooled(Smem<BLK>& sm, const AttnParams& p, int h, int r, int I, int L,
                                             int cb, float kscale, float vscale) {
  const int tid = threadIdx.x;
  const int64_t base = ((int64_t)h * p.NB_tot + p.rt.blk_off[r]) * kHeadDim;
  constexpr int kChunks = BLK * (kHeadDim / 8);
  for (int ci = tid; ci < kChunks; ci += kThreads) {
    const int kk = ci >> 4, dc = ci & 15;
    const int J = cb * BLK + kk;
    uint4 o = make_uint4(0, 0, 0, 0);
    if (J < I) {
      const float4* src = reinterpret_cast<const float4*>(p.k_bar + base + (int64_t)J * kHeadDim + dc * 8);
      const float4 a = src[0], b = src[1];
      o.x = pack_bf16x2(a.x * kscale, a.y * kscale);
      o.y = pack_bf16x2(a.z * kscale, a.w * kscale);
      o.z = pack_bf16x2(b.x * kscale, b.y * kscale);
      o.w = pack_bf16x2(b.z * kscale, b.w * kscale);
    }
    *reinterpret_cast<uint4*>(&sm.k[kk * kKPitch + dc * 8]) = o;
  }
  constexpr int kVTasks = (BLK / 4) * (kHeadDim / 8);
  for (int tk = tid; tk < kVTasks; tk += kThreads) {
    const int dc = tk & 15, kg = tk >> 4;
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int J = cb * BLK + kg * 4 + i;
      v[i] = make_uint4(0, 0, 0, 0);
      if (J < I) {
        const float4* src = reinterpret_cast<const float4*>(p.v_bar + base + (int64_t)J * kHeadDim + dc * 8);
        const float4 a = src[0], b = src[1];
        v[i].x = pack_bf16x2(a.x * vscale, a.y * vscale);
        v[i].y = pack_bf16x2(a.z * vscale, a.w * vscale);
        v[i].z = pack_bf16x2(b.x * vscale, b.y * vscale);
        v[i].w = pack_bf16x2(b.z * vscale, b.w * vscale);
      }
    }
    vt_store4x8<BLK>(sm, kg, dc, v);
  }
  for (int kk = tid; kk < BLK; kk += kThreads) {
    const int J = cb * BLK + kk;
    float bval = -INFINITY;
    if (J < I && !((sm.selbits[J >> 5] >> (J & 31)) & 1u)) bval = __log2f((float)min(BLK, L - J * BLK));
    sm.bias[kk] = bval;
  }
}

// Per-wave state of the online softmax for 32 query rows.
template <int BLK>
struct WaveState {
  bf16x8 qf[kHeadDim / 16];  // B operand of S^T = K Q^T, one per 16-dim step
  f32x16 o[kHeadDim / 32];   // O^T accumulators, one per 32-dim tile
  float m;                   // running max (log2 units)
  float l;                   // this lane's partial row sum
};

// One key block (exact or pooled) for one wave. kt_lim: last 32-key tile that
// is not fully masked; diag: causal mask inside tile kt_lim; use_bias: add
// sm.bias per key column. tq: this lane's query offset inside the block.
template <int BLK>
__device__ __forceinline__ void attend_block(WaveState<BLK>& ws, const Smem<BLK>& sm, int kt_lim, bool diag,
                                             bool use_bias, int tq, float sl2) {
  constexpr int NKT = BLK / 32;
  const int lane = threadIdx.x & 63;
  const int c = lane & 31, hf = lane >> 5;
  f32x16 s[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    if (kt > kt_lim) continue;
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 16; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.k[(kt * 32 + c) * kKPitch + ks * 16 + hf * 8]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ws.qf[ks], acc, 0, 0, 0);
    }
    s[kt] = acc;
  }
  // scale, bias, mask; local max
  float mloc = kNegBig;
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    if (kt > kt_lim) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 bb = make_float4(0.f, 0.f, 0.f, 0.f);
      if (use_bias) bb = *reinterpret_cast<const float4*>(&sm.bias[kt * 32 + i * 8 + hf * 4]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = s[kt][4 * i + j] * sl2;
        if (use_bias) x += (j == 0 ? bb.x : j == 1 ? bb.y : j == 2 ? bb.z : bb.w);
        if (diag && kt == kt_lim) {
          const int key = kt * 32 + i * 8 + hf * 4 + j;
          if (key > tq) x = -INFINITY;
        }
        s[kt][4 * i + j] = x;
        mloc = fmaxf(mloc, x);
      }
    }
  }
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  const float m_new = fmaxf(ws.m, mloc);
  const float corr = __builtin_amdgcn_exp2f(ws.m - m_new);
  ws.m = m_new;
  ws.l *= corr;
  if (__ballot(corr != 1.0f) != 0) {
#pragma unroll
    for (int dt = 0; dt < kHeadDim / 32; ++dt) ws.o[dt] *= corr;
  }
  // probabilities -> bf16 B operands; PV
  float lsum = 0.f;
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    if (kt > kt_lim) continue;
    bf16x8 pf[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      f32x2 pr[4];
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        const float p0 = __builtin_amdgcn_exp2f(s[kt][8 * s2 + t] - m_new);
        const float p1 = __builtin_amdgcn_exp2f(s[kt][8 * s2 + t + 1] - m_new);
        lsum += p0 + p1;
        pr[t / 2] = f32x2{p0, p1};
      }
      const bf16x2 b0 = __builtin_convertvector(pr[0], bf16x2);
      const bf16x2 b1 = __builtin_convertvector(pr[1], bf16x2);
      const bf16x2 b2 = __builtin_convertvector(pr[2], bf16x2);
      const bf16x2 b3 = __builtin_convertvector(pr[3], bf16x2);
      pf[s2] = bf16x8{b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
    }
#pragma unroll
    for (int dt = 0; dt < kHeadDim / 32; ++dt) {
      const uint16_t* vrow = &sm.vt[(dt * 32 + c) * Smem<BLK>::kVPitch + kt * 32 + hf * 4];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + s2 * 16);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + s2 * 16 + 8);
        const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
        const bf16x8 a = __builtin_bit_cast(bf16x8, w);
        ws.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[s2], ws.o[dt], 0, 0, 0);
      }
    }
  }
  ws.l += lsum;
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
  // C(I) = number of (r, I') with I' > I; non-increasing in I. Find the
  // smallest I with C(I) <= pk.
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

template <int BLK, bool FP8>
__global__ __launch_bounds__(kThreads, 1) void attn_kernel(AttnParams p) {
  __shared__ Smem<BLK> sm;
  constexpr int NKT = BLK / 32;
  int I, r, h, sub;
  decode_work(p, I, r, h, sub);
  const ReqTable& rt = p.rt;
  const int L = rt.tok_off[r + 1] - rt.tok_off[r];
  const int nI = min(BLK, L - I * BLK);
  const int64_t row = (int64_t)h * p.NB_tot + rt.blk_off[r] + I;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int c = lane & 31, hf = lane >> 5;
  const int prow0 = sub * kRowsPerWG + w * 32;   // first packed row of this wave
  const bool wave_active = prow0 < p.G * BLK;
  const int g = h * p.G + (wave_active ? prow0 / BLK : 0);
  const int tq0 = prow0 % BLK;
  const int tq = tq0 + c;
  const bool q_valid = wave_active && tq < nI;
  const int64_t tok = (int64_t)rt.tok_off[r] + (int64_t)I * BLK + tq;

  float sl2 = p.sm_scale * kLog2e;
  float kscale = 1.f, vscale = 1.f, oscale = 1.f;
  if constexpr (FP8) {
    const float dq = *p.descale_q, dk = *p.descale_k, dv = *p.descale_v;
    sl2 *= dq * dk;
    kscale = 1.f / dk;
    vscale = 1.f / dv;
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

  // exact blocks: the CSR row, or every causal block in dense mode
  const int n_exact = p.dense ? I + 1 : p.row_ptr[row + 1] - p.row_ptr[row];
  const int32_t* cols = p.dense ? nullptr : p.col_idx + p.row_ptr[row];
  const bool do_corr = p.mean_correction && !p.dense && I > 0;

  if (do_corr) {
    for (int wd = tid; wd <= (I >> 5); wd += kThreads) sm.selbits[wd] = 0u;
    __syncthreads();
    for (int e = tid; e < n_exact; e += kThreads) {
      const int J = cols[e];
      atomicOr(&sm.selbits[J >> 5], 1u << (J & 31));
    }
  }

  KVStage<BLK> st;
  if (n_exact > 0) kv_load<BLK, FP8>(st, p, r, p.dense ? 0 : cols[0], h, L);
  for (int e = 0; e < n_exact; ++e) {
    const int J = p.dense ? e : cols[e];
    __syncthreads();
    kv_store<BLK>(st, sm);
    __syncthreads();
    if (e + 1 < n_exact) kv_load<BLK, FP8>(st, p, r, p.dense ? e + 1 : cols[e + 1], h, L);
    if (wave_active) {
      const bool diag = (J == I);
      const int kt_lim = diag ? (tq0 >> 5) : NKT - 1;
      attend_block<BLK>(ws, sm, kt_lim, diag, false, tq, sl2);
    }
  }

  if (do_corr) {
    const int nchunks = (I + BLK - 1) / BLK;
    for (int cb = 0; cb < nchunks; ++cb) {
      __syncthreads();
      stage_pooled<BLK>(sm, p, h, r, I, L, cb, kscale, vscale);
      __syncthreads();
      if (wave_active) {
        const int ncols = min(BLK, I - cb * BLK);
        attend_block<BLK>(ws, sm, (ncols - 1) >> 5, false, true, tq, sl2);
      }
    }
  }

  if (!wave_active) return;
  const float l_tot = ws.l + __shfl_xor(ws.l, 32);
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

}  // namespace

hipError_t launch_attn(const AttnParams& p, hipStream_t stream) {
  const int64_t wgs = (int64_t)p.Hkv * p.NB_tot * p.subs;
  dim3 grid((unsigned)wgs);
  if (p.B == 128) {
    if (p.fp8) hipLaunchKernelGGL((attn_kernel<128, true>), grid, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((attn_kernel<128, false>), grid, dim3(kThreads), 0, stream, p);
  } else {
    if (p.fp8) hipLaunchKernelGGL((attn_kernel<64, true>), grid, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((attn_kernel<64, false>), grid, dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

int attn_rows_per_wg() { return kRowsPerWG; }

}  // namespace fpv2
