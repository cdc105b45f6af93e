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
// One kernel, no score round trip through HBM and no host round trip
// (select_kernel; a small reset kernel, or the pooling kernel of fp_stage1,
// clears its look-back state first):
//   * Workgroup = 1024 threads (16 waves); it takes the next tile from an
//     atomic ticket. A tile is T consecutive query blocks of one (KV head,
//     request), T = 16 for launches of many rows and 4 for small ones (a
//     short chunk), so that a small launch still spreads over the CUs; tiles
//     are numbered in CSR row order.
//   * Scores on the fp32 matrix cores (v_mfma_f32_16x16x4_f32): every wave
//     holds the tile's pooled queries (padded to 16 rows) as its B operand
//     in registers and multiplies them with its 16 of every 256 key blocks,
//     whose pooled keys it loads straight into registers as the A operand
//     (the next 256 prefetched); lane l handles row / key block l % 16 and
//     head dims 32 (l / 16) .. + 31. A score does not depend on the tile it
//     falls in (the same products in the same order).
//   * Pass 1 takes each row's max over its causal key blocks; the scores stay
//     in LDS when the longest request has at most kCacheCols key blocks, else
//     pass 2 computes them again, 256 key blocks at a time.
//   * Pass 2, one wave per row: keep = z - max >= ln(alpha) or forced; one
//     ballot per 64 key blocks gives 64 keep bits (LDS) and their count.
//   * Decoupled look-back: the tile publishes its keep count, sums its
//     predecessors' counts back to the nearest one that has published its
//     inclusive prefix (64 states per round trip, one per lane), and
//     publishes its own; the exclusive prefix places its rows in the CSR.
//     Predecessors hold lower tickets, so they are running or done and every
//     wait ends.
//   * Compaction: row_ptr of each row, and the kept key-block ids from the
//     bits, ascending (mbcnt prefix per 64-bit word).
#include <mutex>

#include "common.h"
#include "launch.h"

namespace fpv2 {

// Selection workspace of fp_select_blocks_noalloc, for callers that cannot
// allocate: the ticket (first 256 bytes), then kStaticSelectTiles look-back
// words. One copy per GPU, held until the process ends. In host code the name
// stands for no device address: host code uses the per-device pointer that
// static_select_workspace() obtains with hipGetSymbolAddress.
__device__ __align__(256) unsigned char scratch[256 + (size_t)kStaticSelectTiles * 8];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` per device, once looked up

constexpr int kSelThreads = 1024;
constexpr int kSelRows = 16;            // query blocks per tile, at most (the MFMA's 16 rows)
constexpr int kSelCols = 16 * (kSelThreads / 64);  // key blocks per chunk: 16 per wave
constexpr int kCPitch = kCacheCols + 4; // floats per cached score row
constexpr int kBPitch = kSelCols + 4;   // floats per row of a chunk's score buffer (no cache)
static_assert(kSelThreads / 64 >= kSelRows, "one wave per tile row in pass 2");

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

// Look-back state of a tile: flag in the top two bits, count below.
constexpr uint64_t kAgg = 1ull << 62;    // the tile's own keep count
constexpr uint64_t kIncl = 2ull << 62;   // keep count of this and every earlier tile
constexpr uint64_t kValMask = (1ull << 62) - 1;
constexpr int kMaxSpins = 1 << 22;       // about 0.1 s of s_sleep 1

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectParams p) {
  constexpr int kWaves = kSelThreads / 64;
  __shared__ float s_max[kWaves][kSelRows];
  __shared__ int s_ticket, s_excl;
  __shared__ int s_cnt[kSelRows];
  // [scores: T x kCPitch (cache) or two chunk buffers of T x kBPitch][bits: T x bit_words]
  extern __shared__ __align__(16) unsigned char dyn[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int T = p.tile_blocks;
  if (tid == 0) s_ticket = (int)atomicAdd(p.ticket, 1u);
  __syncthreads();
  const int t = s_ticket;
  // A workspace shared by overlapping calls (a misuse) could hand out tickets
  // past the launch; such a workgroup has no tile.
  if (t >= p.ntiles) return;

  // Tile t: KV head, request and first query block.
  const ReqTable& rt = p.rt;
  const int h = t / p.tiles_per_head;
  int rem = t - h * p.tiles_per_head, r = 0;
  for (;;) {
    const int nt = (rt.blk_off[r + 1] - rt.blk_off[r] + T - 1) / T;
    if (rem < nt || r + 1 >= rt.R) break;
    rem -= nt;
    ++r;
  }
  const int i0 = rem * T;
  const int NBq = rt.blk_off[r + 1] - rt.blk_off[r];
  const int NB = rt.kblk_off[r + 1] - rt.kblk_off[r];
  const int qb0 = rt.qb0[r];
  const int nrows = min(T, NBq - i0);
  const int ncols = qb0 + i0 + nrows;  // key blocks 0 .. the last row's diagonal
  const bool dense = request_dense(p, r);
  const bool cache = p.cache_scores;
  float* const cs = reinterpret_cast<float*>(dyn);
  uint64_t* const bits = reinterpret_cast<uint64_t*>(dyn + (cache ? T * kCPitch * 4 : 2 * T * kBPitch * 4));
  const int ri = w;  // the row this wave ballots and compacts (if < nrows)
  const int I = qb0 + i0 + ri;

  int cnt = 0;
  if (!dense) {
    // MFMA lane roles: row n of the tile (B operand) / key block n of the
    // wave's 16 (A operand), k slot g: head dims 32 g .. 32 g + 31.
    const int n = lane & 15, g = lane >> 4;
    f32x4 qv[8];
    {
      const float* qsrc = p.q_bar + ((int64_t)h * p.NBq_tot + rt.blk_off[r] + i0 + n) * kHeadDim + 32 * g;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        qv[u] = n < nrows ? *reinterpret_cast<const f32x4*>(qsrc + 4 * u) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // This lane's pooled-key slice of chunk c: key block c * 256 + 16 w + n,
    // dims 32 g .. + 31 (zeros past the tile's last column).
    const float* ksrc = p.k_bar + ((int64_t)h * p.kpitch + rt.prow_off[r] + 16 * w + n) * kHeadDim + 32 * g;
    f32x4 kv[8];
    auto load_keys = [&](int c) {
      const int J = c * kSelCols + 16 * w + n;
      const float* src = ksrc + (int64_t)c * kSelCols * kHeadDim;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        kv[u] = J < ncols ? *reinterpret_cast<const f32x4*>(src + 4 * u) : f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // tau * (q_bar . k_bar) of key blocks c * 256 + 16 w + 4 g + i (i = 0..3)
    // against row n; the operands are consumed, so the next chunk's keys can
    // be loaded into kv right after.
    auto scores = [&]() {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[u][0], qv[u][0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[u][1], qv[u][1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[u][2], qv[u][2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[u][3], qv[u][3], acc, 0, 0, 0);
      }
      return acc * p.sel_scale;
    };
    float mx_part = -INFINITY;  // row n's max over this lane's key blocks
    float mx = -INFINITY;       // row ri's max (after pass 1)
    // Keep bits of the 64 key blocks c64 * 64 + lane of row ri, from scores at zrow.
    auto decide = [&](int c64, const float* zrow) {
      const int J = c64 * 64 + lane;
      const bool keep = ri < nrows && J <= I && ((zrow[lane] - mx) >= p.log_alpha || forced_keep(p, I, J, NB));
      const uint64_t word = __ballot(keep);
      if (ri < nrows && lane == 0) bits[ri * p.bit_words + c64] = word;
      cnt += __popcll(word);
    };
    const int nch = (ncols + kSelCols - 1) / kSelCols;
    load_keys(0);
    for (int c = 0; c < nch; ++c) {
      const f32x4 z = scores();
      if (c + 1 < nch) load_keys(c + 1);
      const int J0 = c * kSelCols + 16 * w + 4 * g;  // key block of z[0]
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n < nrows && J0 + i <= qb0 + i0 + n) mx_part = fmaxf(mx_part, z[i]);
      if (cache && n < T) *reinterpret_cast<f32x4*>(cs + n * kCPitch + J0) = z;
    }
    mx_part = fmaxf(mx_part, __shfl_xor(mx_part, 16));
    mx_part = fmaxf(mx_part, __shfl_xor(mx_part, 32));
    if (lane < kSelRows) s_max[w][lane] = mx_part;
    __syncthreads();
    if (ri < nrows) {
#pragma unroll
      for (int v = 0; v < kWaves; ++v) mx = fmaxf(mx, s_max[v][ri]);
    }
    if (cache) {
      if (ri < nrows)
        for (int c64 = 0; c64 * 64 < ncols; ++c64) decide(c64, cs + ri * kCPitch + c64 * 64);
    } else {
      // Pass 2 without the cache: each chunk's scores again, through a
      // buffer of T x 256 (two, alternating, so one barrier per chunk).
      load_keys(0);
      for (int c = 0; c < nch; ++c) {
        const f32x4 z = scores();
        if (c + 1 < nch) load_keys(c + 1);
        float* buf = cs + (c & 1) * T * kBPitch;
        if (n < T) *reinterpret_cast<f32x4*>(buf + n * kBPitch + 16 * w + 4 * g) = z;
        __syncthreads();
        if (ri < nrows)
          for (int q = 0; q < kSelCols / 64 && c * kSelCols + q * 64 < ncols; ++q)
            decide(c * (kSelCols / 64) + q, buf + ri * kBPitch + q * 64);
      }
    }
  } else if (ri < nrows) {
    cnt = I + 1;
  }
  if (ri < nrows && lane == 0) s_cnt[ri] = cnt;
  __syncthreads();

  // Decoupled look-back over the tiles before this one, by wave 0: lane l
  // reads the state of tile hi - l, so one round trip covers 64
  // predecessors; the nearest one with an inclusive prefix ends the walk
  // (tiles before the first count as inclusive zeros).
  if (w == 0) {
    int agg = 0;
    for (int k = 0; k < nrows; ++k) agg += s_cnt[k];
    int excl = 0;
    if (t > 0) {
      if (lane == 0)
        __hip_atomic_store(p.status + t, kAgg | (uint64_t)agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // Predecessors always publish; the bound only keeps a misused workspace
      // (states not reset) from hanging the launch.
      int spins = 0;
      for (int hi = t - 1;;) {
        const int j = hi - lane;
        const uint64_t st =
            j >= 0 ? __hip_atomic_load(p.status + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : kIncl;
        const uint64_t f = st & ~kValMask;
        const uint64_t incl = __ballot(f == kIncl);
        const int first = incl ? __builtin_ctzll(incl) : 64;  // nearest inclusive prefix
        const uint64_t need = first >= 63 ? ~0ull : ((2ull << first) - 1);
        if ((__ballot(f == 0) & need) != 0 && ++spins <= kMaxSpins) {
          __builtin_amdgcn_s_sleep(1);
          continue;
        }
        int v = lane <= first ? (int)(st & kValMask) : 0;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
        excl += v;
        if (first < 64 || spins > kMaxSpins) break;
        hi -= 64;
      }
    }
    if (lane == 0) {
      __hip_atomic_store(p.status + t, kIncl | (uint64_t)(excl + agg), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_excl = excl;
      if (t == p.ntiles - 1) p.row_ptr[(int64_t)p.Hkv * p.NBq_tot] = excl + agg;
    }
  }
  __syncthreads();

  // Row offset of row ri and its kept key-block ids, ascending.
  if (ri < nrows) {
    int base = s_excl;
    for (int k = 0; k < ri; ++k) base += s_cnt[k];
    if (lane == 0) p.row_ptr[(int64_t)h * p.NBq_tot + rt.blk_off[r] + i0 + ri] = base;
    int32_t* out = p.col_idx + base;
    if (dense) {
      for (int J = lane; J <= I; J += 64) out[J] = J;
    } else {
      int pos = 0;
      for (int c = 0; c * 64 <= I; ++c) {
        const uint64_t word = bits[ri * p.bit_words + c];
        if ((word >> lane) & 1ull)
          out[pos + __builtin_amdgcn_mbcnt_hi((uint32_t)(word >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)word, 0))] =
              c * 64 + lane;
        pos += __popcll(word);
      }
    }
  }
}

// Clears the ticket and the tiles' look-back states.
__global__ __launch_bounds__(256) void select_reset_kernel(uint32_t* ticket, uint64_t* status, int ntiles) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) *ticket = 0u;
  for (int j = i; j < ntiles; j += gridDim.x * blockDim.x) status[j] = 0ull;
}

}  // namespace

int select_tile_blocks(int64_t rows) { return rows >= 4096 ? kSelRows : 4; }

hipError_t static_select_workspace(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    // With device `dev` current: its copy of the array.
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

size_t select_dyn_lds(int T, int nb_max) {
  const size_t words = (size_t)(nb_max + 63) / 64;
  const size_t scores = nb_max <= kCacheCols ? (size_t)T * kCPitch * 4 : (size_t)2 * T * kBPitch * 4;
  return scores + (size_t)T * words * 8;
}

hipError_t launch_select_reset(const SelectParams& p, hipStream_t stream) {
  const int blocks = p.ntiles / 256 + 1 < 64 ? p.ntiles / 256 + 1 : 64;
  hipLaunchKernelGGL(select_reset_kernel, dim3(blocks), dim3(256), 0, stream, p.ticket, p.status, p.ntiles);
  return hipGetLastError();
}

hipError_t launch_select(const SelectParams& p, hipStream_t stream) {
  const size_t lds = select_dyn_lds(p.tile_blocks, p.rt.nb_max);
  hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                      (int)lds);
  hipLaunchKernelGGL(select_kernel, dim3(p.ntiles), dim3(kSelThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace fpv2
