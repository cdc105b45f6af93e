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
// One kernel (select_kernel; a small reset kernel, or the pooling kernel of
// fp_stage1, clears its ticket and look-back states first):
//   * Tiles: consecutive CSR rows of one (KV head, request) with about equal
//     causal area (rows x key blocks), about one tile per CU, so the tiles of
//     a launch finish together; an early tile holds many short rows, a late
//     one a few long rows. Workgroup = 1024 threads (16 waves); it takes the
//     next ticket (tiles numbered in CSR order).
//   * Scores on the fp32 matrix cores (v_mfma_f32_16x16x4_f32), 16 rows x 16
//     key blocks per unit: the tile's rows in blocks of 16 (B operand, zero
//     rows past the tile), each against its causal key blocks in 16s (A
//     operand); lane l handles row / key block l % 16 and, in MFMA step
//     4 u + e, head dim 16 u + 4 (l / 16) + e (the four lanes of a row read
//     64 contiguous bytes per load). The waves split the tile's units into contiguous
//     runs and request the next unit's pooled keys before multiplying the
//     current one. A score does not depend on the tile or launch it falls in
//     (the same products in the same order), so chunked and whole launches
//     select alike. Tiles start at multiples of 16 rows when two of the
//     widest 16-row blocks fit the cache, so late tiles are whole blocks.
//   * Every score of the tile stays in its LDS score cache, row after row (a
//     row of n causal key blocks takes n rounded up to 4 floats), and each
//     row's max is kept as it is computed. No score goes through HBM, except
//     in a launch of few, long rows (a chunk of a long prompt): there each
//     tile's key blocks are split among `parts` workgroups, which write their
//     scores and row maxima to the workspace; the last to arrive (an atomic
//     count behind a device fence) loads them into its cache and finishes the
//     tile, the others exit.
//   * One wave per row: keep = z - max >= ln(alpha) or forced, one ballot per
//     64 key blocks, and the row's keep count.
//   * Decoupled look-back: the tile publishes its keep count, sums its
//     predecessors' counts back to the nearest one that has published its
//     inclusive prefix (64 states per round trip, one per lane), and
//     publishes its own; the exclusive prefix places its rows in the CSR.
//     Predecessors hold lower tickets, so they are running or done and every
//     wait ends.
//   * Compaction: row_ptr of each row, and the kept key-block ids, ascending
//     (the same keep test again from the cache; mbcnt prefix per ballot).
#include <atomic>
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
std::atomic<bool> g_lds_set[kMaxDevices];  // selection kernel's LDS limit raised on this device

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
// A tile's cache area stays below A + widest unit <= kSelCacheFloats, and
// its rows i0 .. i0 + n - 1 take at least sum_j (j + 4) = n (n + 7) / 2
// floats, so a tile has at most 279 rows.
static_assert(279 * (279 + 7) / 2 < kSelCacheFloats && 280 * (280 + 7) / 2 >= kSelCacheFloats, "tile row bound");
constexpr int kScanRows = 5;  // rows per lane in the one-wave scan of a tile's counts
static_assert(kSelMaxRowsPerTile >= 280 && kSelMaxRowsPerTile <= kScanRows * 64, "tile rows");
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

// Signed-int keys with the order of the floats (no NaNs), for atomic max.
__device__ __forceinline__ int max_key(float f) {
  const int b = __float_as_int(f);
  return b >= 0 ? b : b ^ 0x7fffffff;
}
__device__ __forceinline__ float key_value(int k) { return __int_as_float(k >= 0 ? k : k ^ 0x7fffffff); }

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  return m;
}

// Look-back state of a tile: flag in the top two bits, count below.
constexpr uint64_t kAgg = 1ull << 62;    // the tile's own keep count
constexpr uint64_t kIncl = 2ull << 62;   // keep count of this and every earlier tile
constexpr uint64_t kValMask = (1ull << 62) - 1;
constexpr int kMaxSpins = 1 << 22;       // about 0.1 s of s_sleep 1

template <bool kSplit>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectParams p) {
  __shared__ int s_ticket, s_excl, s_arrived;
  __shared__ int s_tile[3];  // the tile's request, first row and row count
  __shared__ int s_wsum[kSelWaves];
  __shared__ int s_off[kSelMaxRowsPerTile + 1];  // cache offset (floats) of each tile row
  __shared__ int s_cnt[kSelMaxRowsPerTile];      // kept blocks of each row, then its offset in the tile's CSR part
  __shared__ int s_maxk[kSelMaxRowsPerTile];     // row max of the scores (max_key)
  extern __shared__ __align__(16) float cs[];   // score cache: the tile's rows one after another
  // The wave index is uniform: unit and row indices derived from it stay in
  // scalar registers (and the pooled queries are read with scalar loads).
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Wave 1 takes the ticket while wave 0 brings the launch parameters and
  // request 0's table entries into the scalar cache: each first read of a
  // kernel-argument line is a memory round trip, which later phases would
  // otherwise pay one after another (the empty asm statements only need the
  // values in registers).
  if (tid == 64) s_ticket = (int)atomicAdd(p.ticket, 1u);
  if (w == 0) {
    const ReqTable& rt0 = p.rt;
    asm volatile("" ::"s"(p.q_bar), "s"(p.k_bar), "s"(p.row_ptr), "s"(p.col_idx), "s"(p.status));
    asm volatile("" ::"s"(p.tile_area), "s"(p.gran), "s"(p.tiles_per_head), "s"(p.ntiles), "s"(p.parts),
                 "s"(p.part_cols), "s"(p.sel_scale), "s"(p.log_alpha));
    asm volatile("" ::"s"(p.all_keep), "s"(p.min_sparse_len), "s"(p.sink), "s"(p.window), "s"(p.last_n),
                 "s"(p.Hkv), "s"(p.NBq_tot), "s"(p.kpitch));
    asm volatile("" ::"s"(rt0.R), "s"(rt0.blk_off[0]), "s"(rt0.kblk_off[0]), "s"(rt0.qb0[0]), "s"(rt0.prow_off[0]),
                 "s"(rt0.tok_off[0]));
  }
  __syncthreads();
  const int ticket = s_ticket;
  // A workspace shared by overlapping calls (a misuse) could hand out tickets
  // past the launch; such a workgroup has no work.
  if (ticket >= p.ntiles * p.parts) return;
  const int t = ticket / p.parts, part = ticket - t * p.parts;

  // Tile t: KV head, request, and its rows i0 .. i0 + nr - 1. Wave 0 alone
  // decodes it (a chain of 64-bit scalar products: run by all 16 waves it
  // queued on the CU's scalar unit, the last wave done 3 us after the first)
  // and hands the result to the others through LDS.
  const ReqTable& rt = p.rt;
  const int h = t / p.tiles_per_head;
  if (w == 0) {
    const int64_t A = p.tile_area;
    int k = t - h * p.tiles_per_head, r = 0;
    for (;;) {
      const int nt = sel_tiles_in_request(rt.blk_off[r + 1] - rt.blk_off[r], rt.qb0[r], p.gran, A);
      if (k < nt || r + 1 >= rt.R) break;
      k -= nt;
      ++r;
    }
    const int nbq = rt.blk_off[r + 1] - rt.blk_off[r];
    const int nu = (nbq + p.gran - 1) / p.gran;
    const int j0 = p.gran * sel_first_unit((int64_t)k * A, rt.qb0[r], p.gran, nu);
    const int j1 = p.gran * sel_first_unit((int64_t)(k + 1) * A, rt.qb0[r], p.gran, nu);
    if (lane == 0) {
      s_tile[0] = r;
      s_tile[1] = j0;
      s_tile[2] = min(min(j1, nbq) - j0, kSelMaxRowsPerTile);
    }
  }
  __syncthreads();
  const int r = __builtin_amdgcn_readfirstlane(s_tile[0]);
  const int i0 = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int nr = __builtin_amdgcn_readfirstlane(s_tile[2]);
  const int NBq = rt.blk_off[r + 1] - rt.blk_off[r];
  const int NB = rt.kblk_off[r + 1] - rt.kblk_off[r];
  const int qb0 = rt.qb0[r];
  const int I0 = qb0 + i0;  // key block of the tile's first row; row j has I0 + j + 1 causal blocks
  const bool dense = request_dense(p, r);
  if (dense && part != 0) return;  // a dense tile is written by its first part alone

  if (!dense) {
    // Cache offsets: exclusive prefix of the rows' lengths rounded up to 4.
    if (tid < kSelMaxRowsPerTile) {
      int x = tid < nr ? ((I0 + tid + 4) & ~3) : 0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      s_off[tid + 1] = x;
      if (lane == 63) s_wsum[w] = x;
      s_maxk[tid] = max_key(-INFINITY);
    }
    if (tid == 0) s_off[0] = 0;
    __syncthreads();
    if (tid < kSelMaxRowsPerTile) {
      int add = 0;
      for (int v = 0; v < w; ++v) add += s_wsum[v];
      s_off[tid + 1] += add;
    }
    __syncthreads();

    // This workgroup's key blocks: all, or part `part` of the tile's split.
    const int c_lo = kSplit ? part * p.part_cols : 0;
    const int c_hi = kSplit ? c_lo + p.part_cols : INT32_MAX;
    float* const spill = kSplit ? p.spill + (int64_t)t * p.lds_floats : nullptr;
    // Units (row block b of 16 rows, key blocks 16 cb .. 16 cb + 15) in
    // row-block order; row block b needs the causal key blocks of its last row
    // within [c_lo, c_hi).
    const int n = lane & 15, g = lane >> 4;
    const int nrb = (nr + 15) >> 4;
    auto cb_lo = [&](int) { return c_lo / 16; };
    auto cb_hi = [&](int b) { return (min(c_hi, I0 + min(16 * b + 16, nr)) + 15) >> 4; };
    auto units_of = [&](int b) { return max(cb_hi(b) - cb_lo(b), 0); };
    int U = 0;
    for (int b = 0; b < nrb; ++b) U += units_of(b);
    // Contiguous runs of units per wave; with no more units than waves, unit
    // k goes to wave 15 - k, so consecutive units run on different SIMDs
    // (wave w is on SIMD w % 4) rather than queueing on one matrix core, and
    // wave 0, which decodes the tile, gets one last.
    const int wr = kSelWaves - 1 - w;
    const int u_begin = U <= kSelWaves ? min(wr, U) : (int)((int64_t)U * w / kSelWaves);
    const int u_end = U <= kSelWaves ? min(wr + 1, U) : (int)((int64_t)U * (w + 1) / kSelWaves);
    if (u_begin < u_end) {
      // Buffer loads, no branches: lanes past the tile's rows or the
      // request's key blocks read zeros (the descriptors' record bounds).
      const __amdgpu_buffer_rsrc_t qres = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(p.q_bar + ((int64_t)h * p.NBq_tot + rt.blk_off[r] + i0) * kHeadDim), (short)0,
          nr * kHeadDim * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(p.k_bar + ((int64_t)h * p.kpitch + rt.prow_off[r]) * kHeadDim), (short)0,
          NB * kHeadDim * 4, 0x00020000);
      // Lane (n, g) holds head dims 16 u + 4 g .. + 3 of its row / key block
      // in register u: the four lanes of a row read 64 contiguous bytes, so a
      // load instruction touches 16 cache lines (not 64).
      const int lane_off = (n * kHeadDim + 4 * g) * 4;
      auto load_q = [&](f32x4 (&qv)[8], int b) {
        const int off = 16 * b * kHeadDim * 4 + lane_off;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          qv[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(qres, off + 64 * u, 0, 0));
      };
      auto load_k = [&](f32x4 (&kv)[8], int cb) {
        const int off = 16 * cb * kHeadDim * 4 + lane_off;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          kv[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(kres, off + 64 * u, 0, 0));
      };
      f32x4 qv[8], ka[8], kb[8];
      // tau * (q_bar . k_bar) of key blocks 16 cb + 4 g + i (i = 0..3)
      // against row 16 b + n: cached (or spilled) if causal, and the row's
      // running max.
      auto unit = [&](const f32x4 (&kv)[8], int b, int cb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[u][0], qv[u][0], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[u][1], qv[u][1], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[u][2], qv[u][2], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[u][3], qv[u][3], acc, 0, 0, 0);
        }
        const f32x4 z = acc * p.sel_scale;
        const int row = 16 * b + n, J0 = 16 * cb + 4 * g;
        const int lim = I0 + row;  // last causal key block of the row
        if (row < nr && J0 <= lim) {
          if (kSplit)
            *reinterpret_cast<f32x4*>(spill + s_off[row] + J0) = z;
          else
            *reinterpret_cast<f32x4*>(cs + s_off[row] + J0) = z;
        }
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (J0 + i <= lim) m = fmaxf(m, z[i]);
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (g == 0 && row < nr) atomicMax(&s_maxk[row], max_key(m));
      };
      // The wave's units row block by row block; within one, the next key
      // chunk is requested before the current products, so the loop waits
      // only for keys requested one unit earlier (the block's last unit is
      // peeled off: nothing is requested past the wave's units).
      int b = 0, first = u_begin;
      while (first >= units_of(b)) {
        first -= units_of(b);
        ++b;
      }
      for (int u = u_begin; u < u_end; ++b) {
        const int c0 = cb_lo(b) + first;
        const int c_end = min(cb_hi(b), c0 + (u_end - u));
        load_q(qv, b);
        load_k(ka, c0);
        for (int cb = c0; cb + 1 < c_end; ++cb) {
          load_k(kb, cb + 1);
          unit(ka, b, cb);
#pragma unroll
          for (int x = 0; x < 8; ++x) ka[x] = kb[x];
        }
        unit(ka, b, c_end - 1);
        u += c_end - c0;
        first = 0;
      }
    }
    __syncthreads();

    if (kSplit) {
      // Publish this part's row maxima; the last part of the tile to arrive
      // takes every part's scores and maxima into its cache and goes on.
      // The barrier puts every wave's stores in L2; one device-scope fence
      // then releases them before the arrival count, and the last part's
      // fence acquires the others' before the barrier lets its waves read.
      if (tid < nr) p.spill_max[(int64_t)ticket * kSelMaxRowsPerTile + tid] = s_maxk[tid];
      __syncthreads();
      if (tid == 0) {
        __threadfence();
        s_arrived = (int)atomicAdd((unsigned long long*)(p.status + p.ntiles + t), 1ull);
        if (s_arrived == p.parts - 1) __threadfence();
      }
      __syncthreads();
      if (s_arrived != p.parts - 1) return;
      // Eight loads in flight per thread (the parts wrote from other CUs:
      // these come from beyond L2).
      const int n4 = s_off[nr];
      for (int x0 = 4 * tid; x0 < n4; x0 += 8 * 4 * kSelThreads) {
        f32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int x = x0 + j * 4 * kSelThreads;
          if (x < n4) v[j] = *reinterpret_cast<const f32x4*>(spill + x);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int x = x0 + j * 4 * kSelThreads;
          if (x < n4) *reinterpret_cast<f32x4*>(cs + x) = v[j];
        }
      }
      if (tid < nr) {
        const int32_t* pm = p.spill_max + (int64_t)t * p.parts * kSelMaxRowsPerTile + tid;
        int m = max_key(-INFINITY);
        for (int q0 = 0; q0 < p.parts; q0 += 8) {
          int v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = q0 + j < p.parts ? pm[(q0 + j) * kSelMaxRowsPerTile] : m;
#pragma unroll
          for (int j = 0; j < 8; ++j) m = max(m, v[j]);
        }
        s_maxk[tid] = m;
      }
      __syncthreads();
    }

    // Keep counts, one wave per row (four ballots in flight).
    for (int row = w; row < nr; row += kSelWaves) {
      const int I = I0 + row, nc = I + 1;
      const float* zr = cs + s_off[row];
      const float m = key_value(s_maxk[row]);
      int cnt = 0;
      for (int c0 = 0; c0 < nc; c0 += 4 * 64) {
        float z[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int J = c0 + 64 * q + lane;
          z[q] = J < nc ? zr[J] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int J = c0 + 64 * q + lane;
          const bool keep = J < nc && ((z[q] - m) >= p.log_alpha || forced_keep(p, I, J, NB));
          cnt += __popcll(__ballot(keep));
        }
      }
      if (lane == 0) s_cnt[row] = cnt;
    }
  } else {
    for (int row = tid; row < nr; row += kSelThreads) s_cnt[row] = I0 + row + 1;
  }
  __syncthreads();

  // Wave 0: the rows' offsets within the tile (five rows per lane), then the
  // decoupled look-back over the tiles before this one: lane l reads the
  // state of tile hi - l, so one round trip covers 64 predecessors; the
  // nearest one with an inclusive prefix ends the walk (tiles before the
  // first count as inclusive zeros).
  if (w == 0) {
    int c4[kScanRows], loc = 0;
#pragma unroll
    for (int j = 0; j < kScanRows; ++j) {
      const int row = kScanRows * lane + j;
      c4[j] = row < nr ? s_cnt[row] : 0;
      loc += c4[j];
    }
    int x = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    const int agg = __shfl(x, 63);
    int run = x - loc;
#pragma unroll
    for (int j = 0; j < kScanRows; ++j) {
      const int row = kScanRows * lane + j;
      if (row < nr) s_cnt[row] = run;
      run += c4[j];
    }
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

  // Row offsets and the kept key-block ids, ascending, one wave per row.
  const int64_t row0 = (int64_t)h * p.NBq_tot + rt.blk_off[r] + i0;  // CSR row of the tile's first row
  for (int row = w; row < nr; row += kSelWaves) {
    const int I = I0 + row, nc = I + 1;
    const int base = s_excl + s_cnt[row];
    if (lane == 0) p.row_ptr[row0 + row] = base;
    int32_t* out = p.col_idx + base;
    if (dense) {
      for (int J = lane; J < nc; J += 64) out[J] = J;
    } else {
      const float* zr = cs + s_off[row];
      const float m = key_value(s_maxk[row]);
      int pos = 0;
      for (int c0 = 0; c0 < nc; c0 += 4 * 64) {
        float z[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int J = c0 + 64 * q + lane;
          z[q] = J < nc ? zr[J] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int J = c0 + 64 * q + lane;
          const bool keep = J < nc && ((z[q] - m) >= p.log_alpha || forced_keep(p, I, J, NB));
          const uint64_t word = __ballot(keep);
          if (keep)
            out[pos + __builtin_amdgcn_mbcnt_hi((uint32_t)(word >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)word, 0))] =
                J;
          pos += __popcll(word);
        }
      }
    }
  }
}

// Clears the ticket and the state words (look-back states, arrival counts).
__global__ __launch_bounds__(256) void select_reset_kernel(uint32_t* ticket, uint64_t* status, int nwords) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) *ticket = 0u;
  for (int j = i; j < nwords; j += gridDim.x * blockDim.x) status[j] = 0ull;
}

}  // namespace

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

hipError_t launch_select_reset(const SelectParams& p, hipStream_t stream) {
  const int blocks = p.reset_words / 256 + 1 < 64 ? p.reset_words / 256 + 1 : 64;
  hipLaunchKernelGGL(select_reset_kernel, dim3(blocks), dim3(256), 0, stream, p.ticket, p.status, p.reset_words);
  return hipGetLastError();
}

hipError_t launch_select(const SelectParams& p, hipStream_t stream) {
  if (p.lds_floats > kSelCacheFloats || p.parts < 1 || p.parts > kSelMaxParts) return hipErrorInvalidValue;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!g_lds_set[dev].load(std::memory_order_acquire)) {
    // The largest score cache any launch asks for, once per device.
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kSelCacheFloats * 4);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kSelCacheFloats * 4);
    if (e != hipSuccess) return e;
    g_lds_set[dev].store(true, std::memory_order_release);
  }
  const dim3 grid((unsigned)p.ntiles * (unsigned)p.parts);
  if (p.parts > 1)
    hipLaunchKernelGGL(select_kernel<true>, grid, dim3(kSelThreads), (size_t)p.lds_floats * 4, stream, p);
  else
    hipLaunchKernelGGL(select_kernel<false>, grid, dim3(kSelThreads), (size_t)p.lds_floats * 4, stream, p);
  return hipGetLastError();
}

}  // namespace fpv2
