// Host <-> kernel interface of the gfx950 block-sparse prefill library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace fpv2 {

struct PoolParams {
  const void* q;
  const void* k;
  const void* v;
  float* q_bar;
  float* k_bar;
  float* v_bar;
  const float* descale_q;
  const float* descale_k;
  const float* descale_v;
  int32_t Hq, Hkv, G, B, NBq_tot, NBk_tot, fp8;
  int32_t kpitch;       // rows per KV head of k_bar / v_bar (>= NBk_tot)
  int32_t chunk_only;   // 1: pool only key blocks J >= qb0 (grid over query blocks)
  uint32_t* sel_ticket; // non-NULL: workgroup 0 also clears the selection's
  uint64_t* sel_status; //   ticket and sel_words state words (fp_stage1)
  int32_t sel_words;
  KVAddr kv;
  ReqTable rt;
};

constexpr int kStaticSelectTiles = FP_NOALLOC_MAX_SELECT_TILES;  // look-back words of the no-alloc workspace

// Selection tiles. Row i of a request (query block i, at key block qb0 + i)
// has qb0 + i + 1 causal key blocks; its scores take at most qb0 + i + 4
// floats of the tile's LDS score cache (the count rounded up to 4). Rows
// are grouped in units of `gran` rows (16: the matrix-core row block, when
// two of the widest blocks fit the cache; else 1); unit j bounds its cache
// need by gran * (qb0 + gran * (j + 1) + 3) floats. A tile is the units of
// one (KV head, request) whose cache prefix sel_area_before(j) falls in
// [k A, (k + 1) A) for a launch-wide area A: consecutive CSR rows of about
// equal work. A launch of few units also splits each tile's key blocks into
// `parts` ranges of `part_cols`, one workgroup each.
constexpr int kSelCacheFloats = 39936;   // LDS score cache of a tile: A + widest unit <= this (156 KB)
constexpr int kSelTargetTiles = 256;     // workgroups per launch to aim for (one per CU)
constexpr int kSelMaxParts = 64;
constexpr int kSelMaxRowsPerTile = 320;  // bound on a tile's rows (at most 279 by the cache bound)

__host__ __device__ inline int64_t sel_area_before(int64_t j, int64_t qb0, int gran) {
  return (int64_t)gran * (j * (qb0 + gran + 3) + (int64_t)gran * (j * (j - 1) / 2));
}

// Smallest j in [0, nu] with sel_area_before(j) >= a (nu if none).
__host__ __device__ inline int sel_first_unit(int64_t a, int qb0, int gran, int nu) {
  const double al = (double)gran * (qb0 + gran + 3), be = (double)gran * gran;
  const double b = al - 0.5 * be;
  int j = (int)((-b + sqrt(b * b + 2.0 * be * (double)a)) / be);
  j = j < 0 ? 0 : (j > nu ? nu : j);
  while (j < nu && sel_area_before(j, qb0, gran) < a) ++j;
  while (j > 0 && sel_area_before(j - 1, qb0, gran) >= a) --j;
  return j;
}

// Tiles of a request of nbq query blocks: one per multiple of A that the
// cache prefixes of its units reach.
__host__ __device__ inline int sel_tiles_in_request(int nbq, int qb0, int gran, int64_t A) {
  const int nu = (nbq + gran - 1) / gran;
  return nu <= 0 ? 0 : (int)(sel_area_before(nu - 1, qb0, gran) / A) + 1;
}

struct SelectParams {
  const float* q_bar;
  const float* k_bar;
  int32_t* row_ptr;
  int32_t* col_idx;
  uint32_t* ticket;   // workspace: tile ticket (zero before the launch)
  uint64_t* status;   // workspace: look-back state per tile, then (parts > 1) an
                      // arrival count per tile; reset_words words, zero before the launch
  int32_t* spill_max; // workspace (parts > 1): [ntiles * parts][256] row-max keys of each part
  float* spill;       // workspace (parts > 1): [ntiles][lds_floats] the tiles' scores, cache layout
  int64_t tile_area;       // A
  int32_t gran;            // rows per tiling unit (16 or 1)
  int32_t tiles_per_head;  // sum_r sel_tiles_in_request(NBq_r, qb0_r, gran, A)
  int32_t ntiles;          // Hkv * tiles_per_head
  int32_t parts;           // workgroups per tile (1: no key-block split)
  int32_t part_cols;       // key blocks per part, a multiple of 64 (parts > 1)
  int32_t reset_words;     // ntiles, or 2 * ntiles with parts > 1
  int32_t lds_floats;      // dynamic LDS of the launch: A + widest row (<= kSelCacheFloats)
  float sel_scale;
  float log_alpha;    // ln(alpha), fp32
  int32_t all_keep;   // alpha <= 0
  int32_t min_sparse_len;
  int32_t sink, window, last_n;  // forced keeps, in blocks
  int32_t Hkv, NBq_tot, NBk_tot, B;
  int32_t kpitch;     // rows per KV head of k_bar (>= NBk_tot)
  ReqTable rt;
};

struct AttnParams {
  const void* q;
  const void* k;        // caller's K / V (bf16 or FP8 codes)
  const void* v;
  const void* kk;       // K the attention kernel reads: k (bf16 or FP8 codes)
  const void* vv;       // V as bf16: v, or for FP8 the workspace copy of its codes
  const float* k_bar;
  const float* v_bar;
  uint16_t* kbar16;     // workspace: bf16 k_bar / v_bar in code units (or NULL)
  uint16_t* vbar16;
  int64_t kv_elems;     // elements of each of K and V (tokens or page slots x Hkv x d)
  const int32_t* row_ptr;
  const int32_t* col_idx;
  uint16_t* out;        // bf16 bits
  float* lse;
  const float* descale_q;
  const float* descale_k;
  const float* descale_v;
  float sm_scale;
  int32_t Hq, Hkv, G, B, NBq_tot, NBk_tot, T;  // T: query tokens
  int32_t kpitch;       // rows per KV head of k_bar / v_bar (>= NBk_tot)
  int32_t mean_correction;
  int32_t dense;        // 1: ignore the CSR, attend to every causal block
  int32_t subs;         // workgroups per (h, I) row: ceil(G * B / rows_per_wg)
  int32_t splits;       // split-KV parts per row (1: no split)
  float* o_part;        // workspace (splits > 1): [splits, T, Hq, d] normalised partial outputs
  float* lse_part;      // workspace (splits > 1): [splits, T, Hq] partial log2-sum-exps
  int32_t fp8;
  KVAddr kv;
  ReqTable rt;
};

struct CheckParams {
  const int32_t* row_ptr;  // NULL: page table only
  const int32_t* col_idx;
  int64_t cap;             // entries of col_idx
  int32_t* err;
  int32_t rows;            // Hkv * NBq_tot
  int32_t NBq_tot, num_pages;
  KVAddr kv;
  ReqTable rt;
};

size_t pool_lds_bytes(int G);
hipError_t launch_pool(const PoolParams& p, hipStream_t stream);
hipError_t launch_select(const SelectParams& p, hipStream_t stream);
hipError_t launch_select_reset(const SelectParams& p, hipStream_t stream);
// This device's copy of the selection workspace array of the no-alloc entry
// point (looked up once per device, with that device current).
hipError_t static_select_workspace(void** out);
hipError_t launch_attn(const AttnParams& p, hipStream_t stream);
int attn_rows_per_wg();
hipError_t launch_check(const CheckParams& p, hipStream_t stream);

}  // namespace fpv2
