// C ABI of libfpv2.so: argument validation, sizing and kernel launches.
//
// Every entry point validates on the host first and enqueues nothing on
// failure; the library never allocates device memory and never synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/fpv2.h"
#include "launch.h"

using namespace fpv2;

namespace {

thread_local char g_last_error[512] = "";

fp_status fail(fp_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

fp_status ok() {
  g_last_error[0] = '\0';
  return FP_OK;
}

// Host-side shape facts derived from a validated problem.
struct Shape {
  int R;
  int64_t Tq, Tk;
  int64_t NBq_tot, NBk_tot;
  int64_t pairs;  // causal (query block, key block) pairs per KV head
  int nb_max;     // max_r NBk_r
  int64_t kpitch; // rows per KV head of k_bar / v_bar
};

// Key offsets of the problem: cu_seqlens_k, or cu_seqlens for a whole prefill.
const int32_t* key_offsets(const fp_problem* p) { return p->cu_seqlens_k ? p->cu_seqlens_k : p->cu_seqlens; }

fp_status check_problem(const fp_problem* p, Shape* sh) {
  if (!p) return fail(FP_ERR_NULL, "problem is NULL");
  if (p->num_seqs < 1 || p->num_seqs > FP_MAX_SEQS)
    return fail(p->num_seqs < 1 ? FP_ERR_SHAPE : FP_ERR_UNSUPPORTED, "num_seqs=%d outside [1, %d]", p->num_seqs,
                FP_MAX_SEQS);
  if (!p->cu_seqlens) return fail(FP_ERR_NULL, "cu_seqlens (host) is NULL");
  if (p->num_q_heads < 1 || p->num_kv_heads < 1)
    return fail(FP_ERR_SHAPE, "num_q_heads=%d num_kv_heads=%d must be >= 1", p->num_q_heads, p->num_kv_heads);
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(FP_ERR_GQA, "num_q_heads=%d is not a multiple of num_kv_heads=%d", p->num_q_heads, p->num_kv_heads);
  if (p->head_dim != FP_HEAD_DIM) return fail(FP_ERR_UNSUPPORTED, "head_dim=%d (only %d)", p->head_dim, FP_HEAD_DIM);
  if (p->block_size != 64 && p->block_size != 128)
    return fail(FP_ERR_BLOCK, "block_size=%d (64 or 128)", p->block_size);
  if (p->dtype != FP_BF16 && p->dtype != FP_FP8_E4M3) return fail(FP_ERR_DTYPE, "dtype=%d unknown", p->dtype);
  if (p->dtype == FP_FP8_E4M3 && (!p->descale_q || !p->descale_k || !p->descale_v))
    return fail(FP_ERR_DTYPE, "FP8 needs descale_q, descale_k and descale_v");
  const int32_t* cuk = key_offsets(p);
  if (p->cu_seqlens[0] != 0) return fail(FP_ERR_SHAPE, "cu_seqlens[0]=%d must be 0", p->cu_seqlens[0]);
  if (cuk[0] != 0) return fail(FP_ERR_SHAPE, "cu_seqlens_k[0]=%d must be 0", cuk[0]);
  const int B = p->block_size;
  Shape s{};
  s.R = p->num_seqs;
  int64_t nbq_tot = 0, nbk_tot = 0, pairs = 0, tq = 0, tk = 0;
  int nb_max = 0, lk_max = 0;
  for (int r = 0; r < p->num_seqs; ++r) {
    const int64_t Lq = (int64_t)p->cu_seqlens[r + 1] - p->cu_seqlens[r];
    const int64_t Lk = (int64_t)cuk[r + 1] - cuk[r];
    if (Lq < 1) return fail(FP_ERR_SHAPE, "request %d has %lld queries (cu_seqlens must increase)", r, (long long)Lq);
    if (Lk < Lq)
      return fail(FP_ERR_SHAPE, "request %d has %lld keys < %lld queries", r, (long long)Lk, (long long)Lq);
    if ((Lk - Lq) % B != 0)
      return fail(FP_ERR_SHAPE, "request %d: chunk offset %lld is not a multiple of block_size %d", r,
                  (long long)(Lk - Lq), B);
    const int64_t nbk = (Lk + B - 1) / B;
    const int64_t nbq = (Lq + B - 1) / B;
    const int64_t qb0 = (Lk - Lq) / B;
    if (nbk > FP_MAX_BLOCKS_PER_SEQ)
      return fail(FP_ERR_UNSUPPORTED, "request %d has %lld blocks (max %d)", r, (long long)nbk, FP_MAX_BLOCKS_PER_SEQ);
    nbq_tot += nbq;
    nbk_tot += nbk;
    pairs += nbq * qb0 + nbq * (nbq + 1) / 2;
    tq += Lq;
    tk += Lk;
    if (nbk > nb_max) nb_max = (int)nbk;
    if (Lk > lk_max) lk_max = (int)Lk;
  }
  if (tq > INT32_MAX || tk > INT32_MAX) return fail(FP_ERR_UNSUPPORTED, "more than 2^31 tokens");
  s.Tq = tq;
  s.Tk = tk;
  if ((int64_t)p->num_kv_heads * pairs > INT32_MAX)
    return fail(FP_ERR_UNSUPPORTED, "worst-case nnz %lld exceeds int32 CSR offsets",
                (long long)((int64_t)p->num_kv_heads * pairs));
  if (s.Tq * p->num_q_heads > INT32_MAX)
    return fail(FP_ERR_UNSUPPORTED, "Tq * num_q_heads = %lld exceeds int32 LSE indexing",
                (long long)(s.Tq * p->num_q_heads));
  if (p->kv_layout == FP_KV_PAGED) {
    if (!p->page_table) return fail(FP_ERR_NULL, "paged layout needs page_table");
    if (p->page_size < 1) return fail(FP_ERR_LAYOUT, "page_size=%d must be >= 1", p->page_size);
    if (p->num_pages < 1) return fail(FP_ERR_LAYOUT, "num_pages=%d must be >= 1", p->num_pages);
    const int64_t need = ((int64_t)lk_max + p->page_size - 1) / p->page_size;
    if (p->max_pages_per_seq < need)
      return fail(FP_ERR_LAYOUT, "max_pages_per_seq=%d < %lld pages of the longest request", p->max_pages_per_seq,
                  (long long)need);
  } else if (p->kv_layout != FP_KV_CONTIGUOUS) {
    return fail(FP_ERR_LAYOUT, "kv_layout=%d unknown", p->kv_layout);
  }
  if (p->pooled_pitch != 0 && p->pooled_pitch < nbk_tot)
    return fail(FP_ERR_SHAPE, "pooled_pitch=%d < %lld key blocks", p->pooled_pitch, (long long)nbk_tot);
  if (p->pooled_row_off) {
    // Each request's rows [base, base + NBk_r) lie below the pitch, and no
    // two requests' rows overlap (checked on the intervals sorted by base).
    const int64_t pitch = p->pooled_pitch ? p->pooled_pitch : nbk_tot;
    int order[FP_MAX_SEQS];
    int64_t nbk_of[FP_MAX_SEQS];
    for (int r = 0; r < p->num_seqs; ++r) {
      order[r] = r;
      nbk_of[r] = ((int64_t)cuk[r + 1] - cuk[r] + B - 1) / B;
      const int64_t base = p->pooled_row_off[r];
      if (base < 0 || base + nbk_of[r] > pitch)
        return fail(FP_ERR_SHAPE, "pooled_row_off[%d]=%lld: rows up to %lld exceed the pitch %lld", r,
                    (long long)base, (long long)(base + nbk_of[r]), (long long)pitch);
    }
    for (int i = 1; i < p->num_seqs; ++i)  // insertion sort by base (R <= 128)
      for (int j = i; j > 0 && p->pooled_row_off[order[j]] < p->pooled_row_off[order[j - 1]]; --j) {
        const int t = order[j];
        order[j] = order[j - 1];
        order[j - 1] = t;
      }
    for (int i = 1; i < p->num_seqs; ++i) {
      const int a = order[i - 1], b = order[i];
      if ((int64_t)p->pooled_row_off[a] + nbk_of[a] > p->pooled_row_off[b])
        return fail(FP_ERR_SHAPE, "pooled rows of requests %d and %d overlap", a, b);
    }
  }
  s.NBq_tot = nbq_tot;
  s.NBk_tot = nbk_tot;
  s.kpitch = p->pooled_pitch ? p->pooled_pitch : nbk_tot;
  s.pairs = pairs;
  s.nb_max = nb_max;
  if (sh) *sh = s;
  return FP_OK;
}

fp_status check_select(const fp_select_args* a) {
  if (!a) return fail(FP_ERR_NULL, "select args are NULL");
  if (std::isnan(a->alpha)) return fail(FP_ERR_ARG, "alpha is NaN");
  if (!std::isfinite(a->sel_scale) || !(a->sel_scale > 0.f))
    return fail(FP_ERR_ARG, "sel_scale=%g must be finite and > 0", (double)a->sel_scale);
  if (a->min_sparse_len < 0) return fail(FP_ERR_ARG, "min_sparse_len=%d must be >= 0", a->min_sparse_len);
  if (a->sink_blocks < 0 || a->window_blocks < 0 || a->last_n_blocks < 0)
    return fail(FP_ERR_ARG, "sink_blocks=%d window_blocks=%d last_n_blocks=%d must be >= 0", a->sink_blocks,
                a->window_blocks, a->last_n_blocks);
  return FP_OK;
}

fp_status check_attn(const fp_attn_args* a) {
  if (!a) return fail(FP_ERR_NULL, "attention args are NULL");
  if (!std::isfinite(a->sm_scale) || a->sm_scale < 0.f) return fail(FP_ERR_ARG, "sm_scale must be finite and >= 0");
  if (a->mean_correction != 0 && a->mean_correction != 1)
    return fail(FP_ERR_ARG, "mean_correction=%d must be 0 or 1", a->mean_correction);
  if (a->num_splits < 0 || a->num_splits > FP_MAX_SPLITS)
    return fail(FP_ERR_ARG, "num_splits=%d outside [0, %d]", a->num_splits, FP_MAX_SPLITS);
  return FP_OK;
}

// Split-KV parts per row. Automatic: none when the launch already has a
// workgroup for each of the 256 CUs (one resident workgroup per CU); else
// just enough parts to fill them once, at most FP_MAX_SPLITS and at most the
// longest request's key-block count. Each part costs an fp32 partial output
// written and read back, so more parts than that lose time (measured:
// a 128K prompt in 8K chunks on one KV head runs attention 31 % faster with
// 2 parts, and slower again with 8; 8 KV heads, 256 workgroups or more, only
// lose by splitting).
constexpr int64_t kSplitTarget = 256;

int choose_splits(const fp_problem* p, const Shape& s, const fp_attn_args* a) {
  if (a && a->num_splits > 0) return a->num_splits;
  const int G = p->num_q_heads / p->num_kv_heads;
  const int64_t subs = (G * p->block_size + attn_rows_per_wg() - 1) / attn_rows_per_wg();
  const int64_t wgs = (int64_t)p->num_kv_heads * s.NBq_tot * subs;
  if (wgs >= kSplitTarget) return 1;
  int64_t n = (kSplitTarget + wgs - 1) / wgs;
  if (n > FP_MAX_SPLITS) n = FP_MAX_SPLITS;
  if (n > s.nb_max) n = s.nb_max;
  return n < 1 ? 1 : (int)n;
}

ReqTable make_table(const fp_problem* p, const Shape& s) {
  ReqTable t{};
  const int32_t* cuk = key_offsets(p);
  const int B = p->block_size;
  t.R = s.R;
  t.nb_max = s.nb_max;
  t.blk_off[0] = 0;
  t.kblk_off[0] = 0;
  for (int r = 0; r <= s.R; ++r) {
    t.tok_off[r] = p->cu_seqlens[r];
    t.ktok_off[r] = cuk[r];
  }
  for (int r = 0; r < s.R; ++r) {
    const int Lq = p->cu_seqlens[r + 1] - p->cu_seqlens[r];
    const int Lk = cuk[r + 1] - cuk[r];
    t.blk_off[r + 1] = t.blk_off[r] + (Lq + B - 1) / B;
    t.kblk_off[r + 1] = t.kblk_off[r] + (Lk + B - 1) / B;
    t.qb0[r] = (Lk - Lq) / B;
  }
  for (int r = 0; r < s.R; ++r) t.prow_off[r] = p->pooled_row_off ? p->pooled_row_off[r] : t.kblk_off[r];
  return t;
}

KVAddr make_kv(const fp_problem* p) {
  KVAddr a{};
  a.paged = p->kv_layout == FP_KV_PAGED;
  a.page_table = a.paged ? p->page_table : nullptr;
  a.page_size = a.paged ? p->page_size : 1;
  a.max_pages = a.paged ? p->max_pages_per_seq : 0;
  return a;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Selection tiles: consecutive CSR rows of one (KV head, request) whose
// score-cache prefixes fall in one multiple of the launch's area A. Rows go
// in units of 16 (the matrix-core row block) when two of the widest 16-row
// blocks fit the cache, else one by one. A is at least the widest unit (no
// empty tiles) and at most what leaves room for it in the cache; launches
// with enough area make about kSelTargetTiles tiles. A launch of too few
// units for that (a chunk of a long prompt, a short prompt) makes one tile
// per 16-row block and splits each tile's key blocks among up to
// kSelMaxParts workgroups, unless the caller has no room for the split's
// buffers.
struct SelTiles {
  int64_t area;
  int gran;
  int64_t per_head, total;
  int parts, part_cols;
  int lds_floats;
};

// First query block's key-block id of request r (chunked prefill: > 0).
int req_qb0(const fp_problem* p, int r) {
  const int32_t* cuk = key_offsets(p);
  return ((cuk[r + 1] - cuk[r]) - (p->cu_seqlens[r + 1] - p->cu_seqlens[r])) / p->block_size;
}

int64_t req_nbq(const fp_problem* p, int r) {
  return ((int64_t)p->cu_seqlens[r + 1] - p->cu_seqlens[r] + p->block_size - 1) / p->block_size;
}

SelTiles sel_tiles(const fp_problem* p, const Shape& s, bool allow_split) {
  const int gran = 2 * 16 * ((int64_t)s.nb_max + 3) <= kSelCacheFloats ? 16 : 1;
  const int64_t wmax = (int64_t)gran * (s.nb_max + 3);  // cache floats of the widest unit
  int64_t total = 0;
  for (int r = 0; r < p->num_seqs; ++r) {
    const int64_t nu = (req_nbq(p, r) + gran - 1) / gran;
    total += sel_area_before(nu, req_qb0(p, r), gran);
  }
  total *= p->num_kv_heads;
  auto tiles_for = [&](int64_t A) {
    SelTiles st{};
    st.area = A;
    st.gran = gran;
    for (int r = 0; r < p->num_seqs; ++r)
      st.per_head += sel_tiles_in_request((int)req_nbq(p, r), req_qb0(p, r), gran, A);
    st.total = st.per_head * p->num_kv_heads;
    st.parts = 1;
    st.part_cols = 0;
    st.lds_floats = (int)(A + wmax);
    return st;
  };
  const int64_t per_target = (total + kSelTargetTiles - 1) / kSelTargetTiles;
  if (allow_split && gran == 16 && per_target < wmax) {
    // Matrix-core units (16 rows x 16 key blocks) per tile; a tile with more
    // than one per wave splits its key blocks, and then into parts of about 4
    // units (one on each SIMD's matrix core): measured on 2048-token chunks of
    // a 128K prompt, 10 % less Stage 1 time than parts of 16 units, while
    // splitting launches of at most one unit per wave (a 32K prompt) only adds
    // the parts' score round trip.
    const SelTiles st = tiles_for(wmax);
    int64_t units = 0;
    for (int r = 0; r < p->num_seqs; ++r) {
      const int64_t nbq = req_nbq(p, r), qb0 = req_qb0(p, r);
      for (int64_t j = 0; 16 * j < nbq; ++j) units += (qb0 + std::min(16 * j + 16, nbq) + 15) / 16;
    }
    units *= p->num_kv_heads;
    const int64_t by_units = units / (16 * st.total) > 1 ? units / (4 * st.total) : 1;
    const int64_t by_cus = (kSelTargetTiles + st.total - 1) / st.total;
    int parts = (int)std::max<int64_t>(1, std::min<int64_t>(std::min(by_units, by_cus), kSelMaxParts));
    const int cols = (s.nb_max + parts - 1) / parts;
    const int part_cols = (cols + 63) / 64 * 64;
    parts = (s.nb_max + part_cols - 1) / part_cols;
    if (parts > 1) {
      SelTiles sp = st;
      sp.parts = parts;
      sp.part_cols = part_cols;
      return sp;
    }
  }
  return tiles_for(std::min(std::max(per_target, wmax), kSelCacheFloats - wmax));
}

// Selection workspace: the tile ticket (256 bytes), one look-back word per
// tile, and with a key-block split one arrival count per tile, each part's
// row maxima and each tile's scores.
struct WsLayout {
  size_t ticket, status, spill_max, spill, total;
  int reset_words;
};

WsLayout ws_layout(const SelTiles& st) {
  WsLayout w{};
  w.ticket = 0;
  w.status = 256;
  const bool split = st.parts > 1;
  w.reset_words = (int)(st.total * (split ? 2 : 1));
  w.spill_max = w.status + align256((size_t)w.reset_words * sizeof(uint64_t));
  w.spill = w.spill_max + (split ? align256((size_t)st.total * st.parts * kSelMaxRowsPerTile * 4) : 0);
  w.total = w.spill + (split ? align256((size_t)st.total * st.lds_floats * 4) : 0);
  return w;
}

// Attention workspace: bf16 k_bar, v_bar (sparse calls), for FP8 a bf16 copy
// of the V codes in the caller's layout (K is read as FP8), and with split-KV the parts'
// fp32 outputs [splits, Tq, Hq, d] and log2-sum-exps [splits, Tq, Hq].
struct AttnWs {
  size_t kbar16, vbar16, vv, opart, lsepart, total;
  int64_t kv_elems;
  int splits;
};

AttnWs attn_ws_layout(const fp_problem* p, const Shape& s, bool sparse, int splits) {
  AttnWs w{};
  const int64_t kv_rows = p->kv_layout == FP_KV_PAGED ? (int64_t)p->num_pages * p->page_size : s.Tk;
  w.kv_elems = kv_rows * p->num_kv_heads * p->head_dim;
  w.splits = splits;
  const size_t pool = sparse ? align256((size_t)p->num_kv_heads * s.kpitch * p->head_dim * 2) : 0;
  const size_t kv = p->dtype == FP_FP8_E4M3 ? align256((size_t)w.kv_elems * 2) : 0;
  const size_t rows = (size_t)s.Tq * p->num_q_heads;
  const size_t op = splits > 1 ? align256((size_t)splits * rows * p->head_dim * 4) : 0;
  const size_t lp = splits > 1 ? align256((size_t)splits * rows * 4) : 0;
  w.kbar16 = 0;
  w.vbar16 = pool;
  w.vv = 2 * pool;
  w.opart = 2 * pool + kv;
  w.lsepart = w.opart + op;
  w.total = w.lsepart + lp;
  return w;
}

fp_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}


}  // namespace

extern "C" {

fp_status fp_index_shape(const fp_problem* p, int64_t* num_rows, int64_t* max_nnz, int64_t* num_q_blocks,
                         int64_t* num_k_blocks) {
  Shape s;
  fp_status st = check_problem(p, &s);
  if (st) return st;
  if (num_rows) *num_rows = (int64_t)p->num_kv_heads * s.NBq_tot;
  if (max_nnz) *max_nnz = (int64_t)p->num_kv_heads * s.pairs;
  if (num_q_blocks) *num_q_blocks = s.NBq_tot;
  if (num_k_blocks) *num_k_blocks = s.NBk_tot;
  return ok();
}

fp_status fp_select_workspace_bytes(const fp_problem* p, size_t* bytes) {
  Shape s;
  fp_status st = check_problem(p, &s);
  if (st) return st;
  if (!bytes) return fail(FP_ERR_NULL, "bytes is NULL");
  *bytes = ws_layout(sel_tiles(p, s, true)).total;
  return ok();
}

fp_status fp_attn_workspace_bytes(const fp_problem* p, const fp_attn_args* attn, int32_t sparse, size_t* bytes) {
  Shape s;
  fp_status st = check_problem(p, &s);
  if (st) return st;
  if (attn && (st = check_attn(attn))) return st;
  if (!bytes) return fail(FP_ERR_NULL, "bytes is NULL");
  *bytes = attn_ws_layout(p, s, sparse != 0, choose_splits(p, s, attn)).total;
  return ok();
}

fp_status fp_workspace_bytes(const fp_problem* p, int32_t which_call, size_t* bytes) {
  switch (which_call) {
    case FP_CALL_SELECT: return fp_select_workspace_bytes(p, bytes);
    case FP_CALL_SPARSE: return fp_attn_workspace_bytes(p, nullptr, 1, bytes);
    case FP_CALL_DENSE: return fp_attn_workspace_bytes(p, nullptr, 0, bytes);
    default: return fail(FP_ERR_ARG, "fp_workspace_bytes: which_call=%d is not FP_CALL_SELECT, _SPARSE or _DENSE",
                         which_call);
  }
}

fp_status fp_attn_num_splits(const fp_problem* p, const fp_attn_args* attn, int32_t* splits) {
  Shape s;
  fp_status st = check_problem(p, &s);
  if (st) return st;
  if (attn && (st = check_attn(attn))) return st;
  if (!splits) return fail(FP_ERR_NULL, "splits is NULL");
  *splits = choose_splits(p, s, attn);
  return ok();
}

fp_status fp_validate(const fp_problem* p, const fp_select_args* sel, const fp_attn_args* attn) {
  fp_status st = check_problem(p, nullptr);
  if (st) return st;
  if (sel && (st = check_select(sel))) return st;
  if (attn && (st = check_attn(attn))) return st;
  return ok();
}

static fp_status prep_pool(const fp_problem* p, const Shape& s, const void* q, const void* k, const void* v,
                           float* q_bar, float* k_bar, float* v_bar, bool chunk_only, PoolParams* out) {
  if (!q || !k || !v || !q_bar || !k_bar || !v_bar) return fail(FP_ERR_NULL, "pooling: NULL buffer");
  PoolParams pp{};
  pp.q = q; pp.k = k; pp.v = v;
  pp.q_bar = q_bar; pp.k_bar = k_bar; pp.v_bar = v_bar;
  pp.descale_q = p->descale_q; pp.descale_k = p->descale_k; pp.descale_v = p->descale_v;
  pp.Hq = p->num_q_heads; pp.Hkv = p->num_kv_heads; pp.G = p->num_q_heads / p->num_kv_heads;
  pp.B = p->block_size; pp.NBq_tot = (int32_t)s.NBq_tot; pp.NBk_tot = (int32_t)s.NBk_tot;
  pp.fp8 = p->dtype == FP_FP8_E4M3;
  pp.kpitch = (int32_t)s.kpitch;
  pp.chunk_only = chunk_only ? 1 : 0;
  pp.kv = make_kv(p);
  pp.rt = make_table(p, s);
  if (pool_lds_bytes(pp.G) > 64 * 1024) return fail(FP_ERR_UNSUPPORTED, "GQA ratio %d too large for pooling", pp.G);
  *out = pp;
  return FP_OK;
}

static fp_status run_pool(const fp_problem* p, const void* q, const void* k, const void* v, float* q_bar,
                          float* k_bar, float* v_bar, void* stream, bool chunk_only) {
  Shape s;
  fp_status st = check_problem(p, &s);
  if (st) return st;
  PoolParams pp;
  if ((st = prep_pool(p, s, q, k, v, q_bar, k_bar, v_bar, chunk_only, &pp))) return st;
  return hip_status(launch_pool(pp, (hipStream_t)stream), "pool launch");
}

fp_status fp_pool_blocks(const fp_problem* p, const void* q, const void* k, const void* v, float* q_bar,
                         float* k_bar, float* v_bar, void* stream) {
  return run_pool(p, q, k, v, q_bar, k_bar, v_bar, stream, false);
}

fp_status fp_pool_chunk_blocks(const fp_problem* p, const void* q, const void* k, const void* v, float* q_bar,
                               float* k_bar, float* v_bar, void* stream) {
  return run_pool(p, q, k, v, q_bar, k_bar, v_bar, stream, true);
}

// Validates the arguments of a selection call other than its workspace.
static fp_status check_select_call(const fp_problem* p, const Shape& s, const fp_select_args* sel,
                                   const float* q_bar, const float* k_bar, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t col_capacity) {
  fp_status st = check_select(sel);
  if (st) return st;
  if (!q_bar || !k_bar || !row_ptr || !col_idx) return fail(FP_ERR_NULL, "selection: NULL buffer");
  const int64_t max_nnz = (int64_t)p->num_kv_heads * s.pairs;
  if (col_capacity < max_nnz)
    return fail(FP_ERR_CAPACITY, "col_capacity=%lld < max_nnz=%lld", (long long)col_capacity, (long long)max_nnz);
  return FP_OK;
}

// Validates a selection call and fills its kernel parameters (the ticket,
// state words and split buffers in `workspace`). allow_split = false keeps
// every tile in one workgroup (no split buffers).
static fp_status prep_select(const fp_problem* p, const Shape& s, const fp_select_args* sel, const float* q_bar,
                             const float* k_bar, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                             void* workspace, size_t workspace_bytes, bool allow_split, SelectParams* out) {
  fp_status st = check_select_call(p, s, sel, q_bar, k_bar, row_ptr, col_idx, col_capacity);
  if (st) return st;
  const SelTiles tl = sel_tiles(p, s, allow_split);
  if (tl.total * tl.parts > INT32_MAX / 2)
    return fail(FP_ERR_UNSUPPORTED, "%lld selection tiles", (long long)tl.total);
  const WsLayout wl = ws_layout(tl);
  if (!workspace || workspace_bytes < wl.total)
    return fail(FP_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace ? workspace_bytes : (size_t)0,
                wl.total);
  SelectParams sp{};
  sp.q_bar = q_bar; sp.k_bar = k_bar; sp.row_ptr = row_ptr; sp.col_idx = col_idx;
  char* ws = static_cast<char*>(workspace);
  sp.ticket = reinterpret_cast<uint32_t*>(ws + wl.ticket);
  sp.status = reinterpret_cast<uint64_t*>(ws + wl.status);
  sp.spill_max = tl.parts > 1 ? reinterpret_cast<int32_t*>(ws + wl.spill_max) : nullptr;
  sp.spill = tl.parts > 1 ? reinterpret_cast<float*>(ws + wl.spill) : nullptr;
  sp.tile_area = tl.area;
  sp.gran = tl.gran;
  sp.tiles_per_head = (int32_t)tl.per_head;
  sp.ntiles = (int32_t)tl.total;
  sp.parts = tl.parts;
  sp.part_cols = tl.part_cols;
  sp.reset_words = wl.reset_words;
  sp.lds_floats = tl.lds_floats;
  sp.sel_scale = sel->sel_scale;
  sp.all_keep = sel->alpha <= 0.f;
  sp.log_alpha = sel->alpha > 0.f ? (float)std::log((double)sel->alpha) : 0.f;
  sp.min_sparse_len = sel->min_sparse_len;
  sp.sink = sel->sink_blocks;
  sp.window = sel->window_blocks;
  sp.last_n = sel->last_n_blocks;
  sp.Hkv = p->num_kv_heads; sp.NBq_tot = (int32_t)s.NBq_tot; sp.NBk_tot = (int32_t)s.NBk_tot;
  sp.B = p->block_size;
  sp.kpitch = (int32_t)s.kpitch;
  sp.rt = make_table(p, s);
  *out = sp;
  return FP_OK;
}

fp_status fp_select_blocks(const fp_problem* p, const fp_select_args* sel, const float* q_bar, const float* k_bar,
                           int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, void* workspace,
                           size_t workspace_bytes, void* stream) {
  Shape s;
  fp_status st = check_problem(p, &s);
  if (st) return st;
  SelectParams sp;
  if ((st = prep_select(p, s, sel, q_bar, k_bar, row_ptr, col_idx, col_capacity, workspace, workspace_bytes, true,
                        &sp)))
    return st;
  fp_status hs = hip_status(launch_select_reset(sp, (hipStream_t)stream), "select reset launch");
  if (hs) return hs;
  return hip_status(launch_select(sp, (hipStream_t)stream), "select launch");
}

fp_status fp_select_blocks_noalloc(const fp_problem* p, const fp_select_args* sel, const float* q_bar,
                                   const float* k_bar, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                   void* stream) {
  Shape s;
  fp_status st = check_problem(p, &s);
  if (st) return st;
  const SelTiles tl = sel_tiles(p, s, false);
  if (tl.total > FP_NOALLOC_MAX_SELECT_TILES)
    return fail(FP_ERR_CAPACITY, "%lld selection tiles exceed the %d of the no-alloc workspace", (long long)tl.total,
                FP_NOALLOC_MAX_SELECT_TILES);
  // Every argument is checked before the first device call; then this
  // device's array (looked up, not allocated).
  if ((st = check_select_call(p, s, sel, q_bar, k_bar, row_ptr, col_idx, col_capacity))) return st;
  void* ws = nullptr;
  fp_status hs = hip_status(static_select_workspace(&ws), "no-alloc workspace lookup");
  if (hs) return hs;
  SelectParams sp;
  if ((st = prep_select(p, s, sel, q_bar, k_bar, row_ptr, col_idx, col_capacity, ws,
                        256 + (size_t)FP_NOALLOC_MAX_SELECT_TILES * 8, false, &sp)))
    return st;
  hs = hip_status(launch_select_reset(sp, (hipStream_t)stream), "select reset launch");
  if (hs) return hs;
  return hip_status(launch_select(sp, (hipStream_t)stream), "select launch");
}

fp_status fp_stage1(const fp_problem* p, const fp_select_args* sel, int32_t chunk_only, const void* q, const void* k,
                    const void* v, float* q_bar, float* k_bar, float* v_bar, int32_t* row_ptr, int32_t* col_idx,
                    int64_t col_capacity, void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  fp_status st = check_problem(p, &s);
  if (st) return st;
  if (chunk_only != 0 && chunk_only != 1) return fail(FP_ERR_ARG, "chunk_only=%d must be 0 or 1", chunk_only);
  PoolParams pp;
  if ((st = prep_pool(p, s, q, k, v, q_bar, k_bar, v_bar, chunk_only != 0, &pp))) return st;
  SelectParams sp;
  if ((st = prep_select(p, s, sel, q_bar, k_bar, row_ptr, col_idx, col_capacity, workspace, workspace_bytes, true,
                        &sp)))
    return st;
  pp.sel_ticket = sp.ticket;
  pp.sel_status = sp.status;
  pp.sel_words = sp.reset_words;
  fp_status hs = hip_status(launch_pool(pp, (hipStream_t)stream), "pool launch");
  if (hs) return hs;
  return hip_status(launch_select(sp, (hipStream_t)stream), "select launch");
}

static fp_status run_attention(const fp_problem* p, const fp_attn_args* attn, const void* q, const void* k,
                               const void* v, const float* k_bar, const float* v_bar, const int32_t* row_ptr,
                               const int32_t* col_idx, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream, bool dense) {
  Shape s;
  fp_status st = check_problem(p, &s);
  if (st) return st;
  if ((st = check_attn(attn))) return st;
  if (!q || !k || !v || !out) return fail(FP_ERR_NULL, "attention: NULL q/k/v/out");
  if (!dense) {
    if (!row_ptr || !col_idx) return fail(FP_ERR_NULL, "fp_sparse_prefill: NULL CSR");
    if (attn->mean_correction && (!k_bar || !v_bar))
      return fail(FP_ERR_NULL, "fp_sparse_prefill: mean correction needs k_bar and v_bar");
  }
  const AttnWs aw = attn_ws_layout(p, s, !dense, choose_splits(p, s, attn));
  if (aw.total > 0 && (!workspace || workspace_bytes < aw.total))
    return fail(FP_ERR_WORKSPACE, "attention workspace %zu bytes < %zu needed", workspace ? workspace_bytes : (size_t)0,
                aw.total);
  char* ws = static_cast<char*>(workspace);
  AttnParams ap{};
  ap.q = q; ap.k = k; ap.v = v;
  const bool fp8 = p->dtype == FP_FP8_E4M3;
  ap.kk = k;
  ap.vv = fp8 ? static_cast<const void*>(ws + aw.vv) : v;
  ap.kv_elems = aw.kv_elems;
  const bool pooled = !dense && attn->mean_correction;
  ap.kbar16 = pooled ? reinterpret_cast<uint16_t*>(ws + aw.kbar16) : nullptr;
  ap.vbar16 = pooled ? reinterpret_cast<uint16_t*>(ws + aw.vbar16) : nullptr;
  ap.k_bar = k_bar; ap.v_bar = v_bar; ap.row_ptr = row_ptr; ap.col_idx = col_idx;
  ap.out = static_cast<uint16_t*>(out);
  ap.lse = lse;
  ap.descale_q = p->descale_q; ap.descale_k = p->descale_k; ap.descale_v = p->descale_v;
  ap.sm_scale = attn->sm_scale > 0.f ? attn->sm_scale : 1.0f / std::sqrt((float)p->head_dim);
  ap.Hq = p->num_q_heads; ap.Hkv = p->num_kv_heads; ap.G = p->num_q_heads / p->num_kv_heads;
  ap.B = p->block_size; ap.NBq_tot = (int32_t)s.NBq_tot; ap.NBk_tot = (int32_t)s.NBk_tot;
  ap.T = (int32_t)s.Tq;
  ap.kpitch = (int32_t)s.kpitch;
  ap.mean_correction = dense ? 0 : attn->mean_correction;
  ap.dense = dense ? 1 : 0;
  ap.subs = (ap.G * ap.B + attn_rows_per_wg() - 1) / attn_rows_per_wg();
  ap.splits = aw.splits;
  ap.o_part = aw.splits > 1 ? reinterpret_cast<float*>(ws + aw.opart) : nullptr;
  ap.lse_part = aw.splits > 1 ? reinterpret_cast<float*>(ws + aw.lsepart) : nullptr;
  ap.fp8 = p->dtype == FP_FP8_E4M3;
  ap.kv = make_kv(p);
  ap.rt = make_table(p, s);
  return hip_status(launch_attn(ap, (hipStream_t)stream), dense ? "dense attention launch" : "attention launch");
}

fp_status fp_sparse_prefill(const fp_problem* p, const fp_attn_args* attn, const void* q, const void* k,
                            const void* v, const float* k_bar, const float* v_bar, const int32_t* row_ptr,
                            const int32_t* col_idx, void* out, float* lse, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return run_attention(p, attn, q, k, v, k_bar, v_bar, row_ptr, col_idx, out, lse, workspace, workspace_bytes,
                       stream, false);
}

fp_status fp_dense_prefill(const fp_problem* p, const fp_attn_args* attn, const void* q, const void* k,
                           const void* v, void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return run_attention(p, attn, q, k, v, nullptr, nullptr, nullptr, nullptr, out, lse, workspace, workspace_bytes,
                       stream, true);
}

fp_status fp_check_index(const fp_problem* p, const int32_t* row_ptr, const int32_t* col_idx, int64_t col_capacity,
                         int32_t* err, void* stream) {
  Shape s;
  fp_status st = check_problem(p, &s);
  if (st) return st;
  if (!err) return fail(FP_ERR_NULL, "fp_check_index: err is NULL");
  if ((row_ptr == nullptr) != (col_idx == nullptr))
    return fail(FP_ERR_NULL, "fp_check_index: give both row_ptr and col_idx, or neither");
  if (row_ptr && col_capacity < 0)
    return fail(FP_ERR_ARG, "fp_check_index: col_capacity=%lld is negative", (long long)col_capacity);
  CheckParams cp{};
  cp.row_ptr = row_ptr;
  cp.col_idx = col_idx;
  cp.cap = col_capacity;
  cp.err = err;
  cp.rows = (int32_t)((int64_t)p->num_kv_heads * s.NBq_tot);
  cp.NBq_tot = (int32_t)s.NBq_tot;
  cp.num_pages = p->kv_layout == FP_KV_PAGED ? p->num_pages : 0;
  cp.kv = make_kv(p);
  cp.rt = make_table(p, s);
  return hip_status(launch_check(cp, (hipStream_t)stream), "fp_check_index");
}

const char* fp_status_string(fp_status s) {
  switch (s) {
    case FP_OK: return "FP_OK";
    case FP_ERR_NULL: return "FP_ERR_NULL: a required pointer is NULL";
    case FP_ERR_SHAPE: return "FP_ERR_SHAPE: bad sequence lengths, head counts or sizes";
    case FP_ERR_GQA: return "FP_ERR_GQA: num_q_heads is not a multiple of num_kv_heads";
    case FP_ERR_BLOCK: return "FP_ERR_BLOCK: block_size must be 64 or 128";
    case FP_ERR_DTYPE: return "FP_ERR_DTYPE: unknown dtype or missing FP8 descales";
    case FP_ERR_LAYOUT: return "FP_ERR_LAYOUT: bad kv_layout or page arguments";
    case FP_ERR_CAPACITY: return "FP_ERR_CAPACITY: col_idx capacity below worst-case nnz";
    case FP_ERR_WORKSPACE: return "FP_ERR_WORKSPACE: workspace missing or too small";
    case FP_ERR_ARG: return "FP_ERR_ARG: bad scalar argument";
    case FP_ERR_UNSUPPORTED: return "FP_ERR_UNSUPPORTED: outside what this library implements";
    case FP_ERR_HIP: return "FP_ERR_HIP: HIP runtime error";
    default: return "unknown fp_status";
  }
}

const char* fp_last_error(void) { return g_last_error; }

int32_t fp_abi_version(void) { return FPV2_ABI_VERSION; }

}  // extern "C"
