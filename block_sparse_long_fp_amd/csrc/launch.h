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
  uint64_t* sel_status; //   ticket and sel_ntiles look-back states (fp_stage1)
  int32_t sel_ntiles;
  KVAddr kv;
  ReqTable rt;
};

constexpr int kCacheCols = 1024;  // selection scores stay in LDS up to this many key blocks per request
constexpr int kStaticSelectTiles = FP_NOALLOC_MAX_SELECT_TILES;  // look-back words of the no-alloc workspace

struct SelectParams {
  const float* q_bar;
  const float* k_bar;
  int32_t* row_ptr;
  int32_t* col_idx;
  uint32_t* ticket;   // workspace: tile ticket (zero before the launch)
  uint64_t* status;   // workspace: look-back state per tile (zero before the launch)
  int32_t tile_blocks;     // T: query blocks per tile (4, 8 or 16)
  int32_t tiles_per_head;  // sum_r ceil(NBq_r / T)
  int32_t ntiles;          // Hkv * tiles_per_head
  int32_t bit_words;       // 64-bit keep words per tile row: ceil(nb_max / 64)
  int32_t cache_scores;    // nb_max <= kCacheCols: scores kept in LDS between the passes
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

size_t pool_lds_bytes(int G);
hipError_t launch_pool(const PoolParams& p, hipStream_t stream);
hipError_t launch_select(const SelectParams& p, hipStream_t stream);
hipError_t launch_select_reset(const SelectParams& p, hipStream_t stream);
int select_tile_blocks(int64_t rows);      // T for a launch of this many CSR rows
// This device's copy of the selection workspace array of the no-alloc entry
// point (looked up once per device, with that device current).
hipError_t static_select_workspace(void** out);
size_t select_dyn_lds(int T, int nb_max);  // dynamic LDS bytes of the selection kernel
hipError_t launch_attn(const AttnParams& p, hipStream_t stream);
int attn_rows_per_wg();

}  // namespace fpv2
