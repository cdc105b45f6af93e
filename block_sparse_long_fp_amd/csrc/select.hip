// Stage 1b: block scoring, max-based dynamic threshold and CSR compaction.
//
// Method: "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context LLM
// Serving" (metallab.ai paper digest): the abstract's max-based dynamic
// thresholding, Table 9 (alpha sets how many blocks survive) and Table 7 (the
// index is a CSR of selected blocks per KV head, int32 block ids). The
// nestfrontier.com article "128K context now demands Hopper hardware", section
// "A serving setup you can actually test", names the threshold and the minimum
// sparse query length knobs.
//
// Row (h, i) of request r is query block i of the call, at key block
// I = qb0 + i of the request (qb0 > 0 in chunked prefill). It scores every
// causal key block J <= I with
// z_J = tau * q_bar[h,I] . k_bar[h,J] (fp32), takes the row max m, and keeps J
// iff z_J - m >= ln(alpha) (the same as exp(z_J - m) >= alpha), plus the
// forced blocks (the diagonal, and optionally sink / window / last-n rows).
//
// Four kernels, no host round trip:
//   score_kernel    one workgroup per (KV head, tile of 32 query blocks of one
//                   request, tile of 64 key blocks): both pooled tiles staged
//                   in LDS as fp32, each thread computes a 2 x 4 block of
//                   scores, every score summed over the head dim in the same
//                   order (so a score does not depend on its tile), and z goes
//                   to the workspace. Tiles wholly above the diagonal exit.
//   rowstat_kernel  one wave per row: row max of z, then the keep count.
//   scan_kernel     one workgroup: exclusive prefix sum of the row counts
//                   into row_ptr (wave shuffles, then a carry across chunks).
//   compact_kernel  one wave per row: ballot of the keep flags of 64 columns,
//                   mbcnt prefix, ascending column ids written at row_ptr.
#include "common.h"
#include "launch.h"

namespace fpv2 {

namespace {

constexpr int kTileI = 32;       // query blocks per score tile
constexpr int kTileJ = 64;       // key blocks per score tile
constexpr int kScoreThreads = 256;
constexpr int kPad = kHeadDim + 4;

// Scores of request r start at pair_offset(r) in a KV head's z slab; row i of
// the request starts i * qb0 + i (i + 1) / 2 later (row i has qb0 + i + 1).
__device__ __forceinline__ int64_t pair_offset(const ReqTable& rt, int r) {
  int64_t s = 0;
  for (int q = 0; q < r; ++q) {
    const int64_t nb = rt.blk_off[q + 1] - rt.blk_off[q];
    s += nb * rt.qb0[q] + nb * (nb + 1) / 2;
  }
  return s;
}

__device__ __forceinline__ int64_t row_pair_offset(int i, int qb0) {
  return (int64_t)i * qb0 + (int64_t)i * (i + 1) / 2;
}

// Blocks kept whatever their score: the diagonal, the attention sink (the
// first p.sink blocks), the local window (p.window blocks left of the
// diagonal) and every causal block of the last p.last_n blocks of the
// sequence so far, NB = NBk ([article] --flashprefill-attention-sink,
// --flashprefill-window, --flashprefill-last-n-blocks; counts in blocks).
__device__ __forceinline__ bool forced_keep(const SelectParams& p, int I, int J, int NB) {
  return J == I || J < p.sink || J >= I - p.window || I >= NB - p.last_n;
}

__device__ __forceinline__ bool request_dense(const SelectParams& p, int r) {
  const int L = p.rt.tok_off[r + 1] - p.rt.tok_off[r];
  return p.all_keep || L < p.min_sparse_len;
}

__global__ __launch_bounds__(kScoreThreads) void score_kernel(SelectParams p) {
  __shared__ float qs[kTileI][kPad];
  __shared__ float ks[kTileJ][kPad];
  const ReqTable& rt = p.rt;
  const int h = blockIdx.z;
  // Map blockIdx.x to (request, query tile): tiles are numbered request by request.
  int r = 0, tile = blockIdx.x;
  for (;;) {
    const int nb = rt.blk_off[r + 1] - rt.blk_off[r];
    const int nt = (nb + kTileI - 1) / kTileI;
    if (tile < nt || r + 1 >= rt.R) break;
    tile -= nt;
    ++r;
  }
  const int NBq = rt.blk_off[r + 1] - rt.blk_off[r];
  const int NB = rt.kblk_off[r + 1] - rt.kblk_off[r];
  const int qb0 = rt.qb0[r];
  const int i0 = tile * kTileI;
  const int J0 = blockIdx.y * kTileJ;
  // Rows i0 .. i0 + 31 need columns J <= qb0 + i (and J < NB).
  const int i_last = min(NBq, i0 + kTileI) - 1;
  if (i0 >= NBq || J0 > qb0 + i_last || request_dense(p, r)) return;
  const int tid = threadIdx.x;

  const float* qsrc = p.q_bar + ((int64_t)h * p.NBq_tot + rt.blk_off[r]) * kHeadDim;
  const float* ksrc = p.k_bar + ((int64_t)h * p.kpitch + rt.prow_off[r]) * kHeadDim;
  for (int e = tid; e < kTileI * (kHeadDim / 4); e += kScoreThreads) {
    const int rr = e / (kHeadDim / 4), c4 = e % (kHeadDim / 4);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i0 + rr < NBq) v = reinterpret_cast<const float4*>(qsrc + (int64_t)(i0 + rr) * kHeadDim)[c4];
    *reinterpret_cast<float4*>(&qs[rr][c4 * 4]) = v;
  }
  for (int e = tid; e < kTileJ * (kHeadDim / 4); e += kScoreThreads) {
    const int rr = e / (kHeadDim / 4), c4 = e % (kHeadDim / 4);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (J0 + rr < NB) v = reinterpret_cast<const float4*>(ksrc + (int64_t)(J0 + rr) * kHeadDim)[c4];
    *reinterpret_cast<float4*>(&ks[rr][c4 * 4]) = v;
  }
  __syncthreads();

  // Thread (ri, cj) owns rows ri, ri + 16 and columns cj + 16 u, u = 0..3.
  const int ri = tid >> 4, cj = tid & 15;
  float acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[a][u] = 0.f;
#pragma unroll 4
  for (int c = 0; c < kHeadDim; c += 4) {
    float4 qv[2], kv[4];
#pragma unroll
    for (int a = 0; a < 2; ++a) qv[a] = *reinterpret_cast<const float4*>(&qs[ri + 16 * a][c]);
#pragma unroll
    for (int u = 0; u < 4; ++u) kv[u] = *reinterpret_cast<const float4*>(&ks[cj + 16 * u][c]);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[a][u] = fmaf(qv[a].x, kv[u].x, acc[a][u]);
        acc[a][u] = fmaf(qv[a].y, kv[u].y, acc[a][u]);
        acc[a][u] = fmaf(qv[a].z, kv[u].z, acc[a][u]);
        acc[a][u] = fmaf(qv[a].w, kv[u].w, acc[a][u]);
      }
  }
  float* zh = p.zbuf + (int64_t)h * p.pairs_tot + pair_offset(rt, r);
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int i = i0 + ri + 16 * a;
    if (i >= NBq) continue;
    float* zrow = zh + row_pair_offset(i, qb0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int J = J0 + cj + 16 * u;
      if (J <= qb0 + i) zrow[J] = p.sel_scale * acc[a][u];
    }
  }
}

constexpr int kRowThreads = 256;

// Row max and keep count of every row, one wave per row, from the stored
// scores (so the count sees exactly the values the compaction will).
__global__ __launch_bounds__(kRowThreads) void rowstat_kernel(SelectParams p) {
  const ReqTable& rt = p.rt;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kRowThreads / 64) + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)p.Hkv * p.NBq_tot;
  if (row >= rows) return;
  const int h = (int)(row / p.NBq_tot);
  const int b = (int)(row % p.NBq_tot);
  int r = 0;
  while (r + 1 < rt.R && rt.blk_off[r + 1] <= b) ++r;
  const int i = b - rt.blk_off[r];
  const int I = rt.qb0[r] + i;
  const int NB = rt.kblk_off[r + 1] - rt.kblk_off[r];
  if (request_dense(p, r)) {
    if (lane == 0) p.counts[row] = I + 1;
    return;
  }
  const float* zrow = p.zbuf + (int64_t)h * p.pairs_tot + pair_offset(rt, r) + row_pair_offset(i, rt.qb0[r]);
  float m = -INFINITY;
  for (int J = lane; J <= I; J += 64) m = fmaxf(m, zrow[J]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  int cnt = 0;
  for (int J0 = 0; J0 <= I; J0 += 64) {
    const int J = J0 + lane;
    const bool keep = (J <= I) && (((zrow[J] - m) >= p.log_alpha) || forced_keep(p, I, J, NB));
    cnt += __popcll(__ballot(keep));
  }
  if (lane == 0) {
    p.counts[row] = cnt;
    p.rowmax[row] = m;
  }
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ row_ptr, int64_t rows) {
  __shared__ int32_t wsum[kScanThreads / 64];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) {
    carry_s = 0;
    row_ptr[0] = 0;
  }
  __syncthreads();
  for (int64_t base = 0; base < rows; base += kScanThreads) {
    const int64_t i = base + tid;
    int32_t x = i < rows ? counts[i] : 0;
    // inclusive wave scan
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int32_t before = 0;
    for (int k = 0; k < w; ++k) before += wsum[k];
    const int32_t carry = carry_s;
    if (i < rows) row_ptr[i + 1] = carry + before + x;
    __syncthreads();
    if (tid == kScanThreads - 1) carry_s = carry + before + x;
    __syncthreads();
  }
}

constexpr int kCompactThreads = 256;

__global__ __launch_bounds__(kCompactThreads) void compact_kernel(SelectParams p) {
  const ReqTable& rt = p.rt;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kCompactThreads / 64) + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)p.Hkv * p.NBq_tot;
  if (row >= rows) return;
  const int h = (int)(row / p.NBq_tot);
  const int b = (int)(row % p.NBq_tot);
  int r = 0;
  while (r + 1 < rt.R && rt.blk_off[r + 1] <= b) ++r;
  const int i = b - rt.blk_off[r];
  const int I = rt.qb0[r] + i;
  const int NB = rt.kblk_off[r + 1] - rt.kblk_off[r];
  int32_t* out = p.col_idx + p.row_ptr[row];
  if (request_dense(p, r)) {
    for (int J = lane; J <= I; J += 64) out[J] = J;
    return;
  }
  const float* zrow = p.zbuf + (int64_t)h * p.pairs_tot + pair_offset(rt, r) + row_pair_offset(i, rt.qb0[r]);
  const float m = p.rowmax[row];
  int base = 0;
  for (int J0 = 0; J0 <= I; J0 += 64) {
    const int J = J0 + lane;
    const bool keep = (J <= I) && (((zrow[J] - m) >= p.log_alpha) || forced_keep(p, I, J, NB));
    const uint64_t mask = __ballot(keep);
    const int pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
    if (keep) out[base + pre] = J;
    base += __popcll(mask);
  }
}

}  // namespace

hipError_t launch_select(const SelectParams& p, hipStream_t stream) {
  int tiles = 0;
  for (int r = 0; r < p.rt.R; ++r) {
    const int nb = p.rt.blk_off[r + 1] - p.rt.blk_off[r];
    tiles += (nb + kTileI - 1) / kTileI;
  }
  const int jtiles = (p.rt.nb_max + kTileJ - 1) / kTileJ;
  hipLaunchKernelGGL(score_kernel, dim3(tiles, jtiles, p.Hkv), dim3(kScoreThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)p.Hkv * p.NBq_tot;
  const int64_t row_wgs = (rows + (kRowThreads / 64) - 1) / (kRowThreads / 64);
  hipLaunchKernelGGL(rowstat_kernel, dim3((unsigned)row_wgs), dim3(kRowThreads), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, p.counts, p.row_ptr, rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t wgs = (rows + (kCompactThreads / 64) - 1) / (kCompactThreads / 64);
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)wgs), dim3(kCompactThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fpv2
