/*
 * fpv2.h - C ABI of the MI355X (gfx950) mean-corrected block-sparse causal
 * prefill library (libfpv2.so).
 *
 * The method is FlashPrefill V2 as described in "FlashPrefill V2: Block-Sparse
 * Prefill Attention for Long-Context LLM Serving" (paper digest on
 * metallab.ai; cited below as [digest]), in the nestfrontier.com article
 * "128K context now demands Hopper hardware" (cited as [article]) and in the
 * ResearchPod episode on FlashPrefill V2 (researchpod.app; [podcast]).
 *
 * The prefill runs as three calls, in order, on one HIP stream:
 *   1. fp_pool_blocks     block-mean statistics of Q (GQA-packed), K and V
 *                         ([digest] Figure 3, Stage 1; Figure 4 means).
 *   2. fp_select_blocks   max-based dynamic threshold over pooled scores and a
 *                         CSR index of kept blocks ([digest] abstract,
 *                         Table 7 "CSR of selected blocks, per KV head").
 *   3. fp_sparse_prefill  exact online-softmax attention over the kept blocks,
 *                         with the mean-correction surrogate of every pruned
 *                         causal block merged into the same softmax
 *                         ([digest] Figure 3 Stage 2, Figure 4).
 * fp_stage1 runs steps 1 and 2 together in two kernels ([digest] Figure 3:
 * Stage 1 pools and produces the CSR index in one fused pass).
 * fp_dense_prefill is the dense causal comparator built from the same kernels.
 *
 * Conventions shared by every call
 * --------------------------------
 * Memory:    every buffer is allocated and freed by the caller. Pointers marked
 *            DEVICE are HIP device pointers; HOST pointers are read during the
 *            call only. The library never allocates, never synchronises the
 *            stream and keeps no pointer after returning.
 * Streams:   `stream` is a hipStream_t passed as void* (NULL = the null
 *            stream). All device work is enqueued on it, in call order; a call
 *            returns before the work runs.
 * Errors:    every call validates its arguments on the host before enqueuing
 *            anything; on failure it returns a non-zero fp_status, enqueues no
 *            work and writes no output. fp_last_error() then holds a message
 *            (per calling thread). A failed kernel launch returns FP_ERR_HIP.
 * Layouts:   Hq / Hkv query / KV heads, G = Hq / Hkv, d = head_dim (128),
 *            B = block_size.
 *            Request r has Lk_r keys (its sequence so far) and Lq_r <= Lk_r
 *            queries, which are its LAST Lq_r tokens: query t (0-based in the
 *            call) sits at sequence position off_r + t, off_r = Lk_r - Lq_r,
 *            and attends to keys 0 .. off_r + t. Lq_r comes from cu_seqlens,
 *            Lk_r from cu_seqlens_k (NULL: Lk_r = Lq_r, a whole prefill).
 *            off_r > 0 is chunked prefill ([digest] Table 6: serving with 8K and
 *            16K prefill chunks; [podcast]: block scoring runs once per chunk);
 *            off_r must be a multiple of B, so the chunk's query blocks
 *            coincide with key blocks.
 *            Blocks restart at each request's token 0: key block J covers
 *            positions [J*B, min((J+1)*B, Lk_r)), NBk_r = ceil(Lk_r / B); query
 *            block i of the call is key block I = off_r / B + i, i < NBq_r =
 *            ceil(Lq_r / B). Tq = sum_r Lq_r, Tk = sum_r Lk_r; blk_off[r] =
 *            sum_{r'<r} NBq_r', kblk_off[r] = sum_{r'<r} NBk_r', NBq_tot and
 *            NBk_tot the totals.
 *            Q, O:          [Tq, Hq, d] row-major; query head g uses KV head g / G.
 *            K, V contiguous: [Tk, Hkv, d], request r at rows cu_seqlens_k[r] ..
 *            K, V paged:    [num_pages, page_size, Hkv, d]; position t of request r
 *                           is slot t % page_size of page
 *                           page_table[r * max_pages_per_seq + t / page_size]
 *                           ([digest] "What they did", Fix 3; Table 7: paged KV,
 *                           arbitrary page size).
 *            pooled q_bar:  fp32 [Hkv, NBq_tot, d], row h * NBq_tot + blk_off[r] + i.
 *            pooled k_bar, v_bar: fp32 [Hkv, P, d], row h * P + base_r + J,
 *                           P = pooled_pitch (NBk_tot when 0), base_r =
 *                           pooled_row_off[r] (kblk_off[r] when NULL).
 *            CSR:           one row per (h, r, i), row id h * NBq_tot + blk_off[r] + i;
 *                           row_ptr int32 [Hkv * NBq_tot + 1]; col_idx int32
 *                           request-local key-block ids J <= I, strictly
 *                           ascending in a row, the diagonal I always present.
 *            LSE:           fp32 [Hq, Tq], natural log of the full softmax
 *                           denominator (exact terms plus surrogates).
 *            O:             bf16 for both input dtypes.
 */
#ifndef FPV2_H
#define FPV2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FPV2_ABI_VERSION 11

/* Status codes. */
typedef int32_t fp_status;
enum {
  FP_OK = 0,
  FP_ERR_NULL = 1,        /* a required pointer is NULL                          */
  FP_ERR_SHAPE = 2,       /* bad sequence lengths, head counts or sizes          */
  FP_ERR_GQA = 3,         /* num_q_heads is not a multiple of num_kv_heads       */
  FP_ERR_BLOCK = 4,       /* block_size is not 64 or 128                         */
  FP_ERR_DTYPE = 5,       /* unknown dtype, or FP8 without its three descales    */
  FP_ERR_LAYOUT = 6,      /* unknown kv_layout or inconsistent page arguments    */
  FP_ERR_CAPACITY = 7,    /* col_idx capacity below the worst-case nnz           */
  FP_ERR_WORKSPACE = 8,   /* workspace NULL or below fp_*_workspace_bytes      */
  FP_ERR_ARG = 9,         /* bad scalar argument (NaN alpha, sel_scale, sm_scale) */
  FP_ERR_UNSUPPORTED = 10,/* valid request outside this library (head_dim != 128, */
                          /* more than FP_MAX_SEQS requests, too many blocks)    */
  FP_ERR_HIP = 11         /* a HIP runtime call or kernel launch failed          */
};

/* Element type of Q, K and V. FP8 is OCP E4M3 (max 448) with one fp32 descale
 * per tensor: value = code * descale ([digest] "What they did", Fix 2). */
enum { FP_BF16 = 0, FP_FP8_E4M3 = 1 };

/* K/V storage. */
enum { FP_KV_CONTIGUOUS = 0, FP_KV_PAGED = 1 };

/* Limits of this library. */
#define FP_MAX_SEQS 128               /* requests per call                      */
#define FP_MAX_BLOCKS_PER_SEQ 16384   /* NBk_r; 2M tokens at B = 128            */
#define FP_HEAD_DIM 128

/* Problem description shared by all calls. */
typedef struct fp_problem {
  int32_t num_seqs;              /* R, 1 .. FP_MAX_SEQS                           */
  const int32_t* cu_seqlens;     /* HOST [R+1] query offsets; [0] = 0, each Lq_r >= 1 */
  int32_t num_q_heads;           /* Hq >= 1                                        */
  int32_t num_kv_heads;          /* Hkv >= 1, Hq % Hkv == 0                        */
  int32_t head_dim;              /* d, must be 128                                 */
  int32_t block_size;            /* B in {64, 128}: query block = key block        */
  int32_t dtype;                 /* FP_BF16 or FP_FP8_E4M3                         */
  const float* descale_q;        /* DEVICE fp32 scalar; required for FP8, else NULL */
  const float* descale_k;
  const float* descale_v;
  int32_t kv_layout;             /* FP_KV_CONTIGUOUS or FP_KV_PAGED                */
  const int32_t* page_table;     /* DEVICE int32 [R, max_pages_per_seq] (paged)    */
  int32_t page_size;             /* tokens per page, >= 1 (paged)                  */
  int32_t max_pages_per_seq;     /* row pitch of page_table, >= ceil(Lk_r/page_size) */
  int32_t num_pages;             /* pages in each of the K and V pools (paged)     */
  const int32_t* cu_seqlens_k;   /* HOST [R+1] key offsets, or NULL (= cu_seqlens);  */
                                 /* Lk_r >= Lq_r and (Lk_r - Lq_r) % B == 0          */
  int32_t pooled_pitch;          /* rows per KV head of k_bar / v_bar: 0 means      */
                                 /* NBk_tot, else >= NBk_tot (a buffer sized for a  */
                                 /* whole prompt, reused across its chunks)         */
  const int32_t* pooled_row_off; /* HOST [R] first k_bar / v_bar row (per KV head)  */
                                 /* of each request, or NULL (= kblk_off[r]). Rows  */
                                 /* base_r .. base_r + NBk_r - 1 must lie below the */
                                 /* pitch and not overlap another request's. With a */
                                 /* region per request sized for its whole prompt,  */
                                 /* a batch of chunked requests keeps each request's */
                                 /* pooled rows in place from chunk to chunk        */
} fp_problem;

/* Block selection ([digest] abstract: max-based dynamic thresholding;
 * [article] flags --flashprefill-abs-threshold and -min-sparse-q-len).
 * Row (h, I) scores z_J = sel_scale * q_bar[h,I] . k_bar[h,J] for J <= I and
 * keeps J iff exp(z_J - max_J z_J) >= alpha, plus the forced blocks: the
 * diagonal J = I always, and ([article] flags --flashprefill-attention-sink,
 * --flashprefill-window, --flashprefill-last-n-blocks; all counted in blocks,
 * 0 = off) J < sink_blocks, J >= I - window_blocks, and every J <= I when I is
 * one of the last last_n_blocks blocks of the sequence so far (I >= NBk_r -
 * last_n_blocks; in chunked prefill, the chunk's last blocks). */
typedef struct fp_select_args {
  float alpha;                   /* threshold; alpha <= 0 keeps every causal block */
  float sel_scale;               /* score temperature tau, finite and > 0          */
  int32_t min_sparse_len;        /* requests with Lq_r < this keep every causal block */
  int32_t sink_blocks;           /* >= 0 */
  int32_t window_blocks;         /* >= 0 */
  int32_t last_n_blocks;         /* >= 0 */
} fp_select_args;

/* Attention ([digest] Figures 3-4). */
typedef struct fp_attn_args {
  float sm_scale;                /* softmax scale; 0 means 1/sqrt(head_dim)        */
  int32_t mean_correction;       /* 1: each pruned causal block J < I adds the     */
                                 /* logit sm*q.k_bar_J + ln n_J on value v_bar_J;  */
                                 /* 0: pruned blocks are dropped (the ablation)    */
  int32_t num_splits;            /* split-KV parts per row ([digest] Table 7:      */
                                 /* count-balanced CSR splits), 0 .. FP_MAX_SPLITS; */
                                 /* 0 = chosen from the problem's size (more parts */
                                 /* when a launch has few rows), 1 = no split      */
} fp_attn_args;

#define FP_MAX_SPLITS 16

/* Host-only queries (no GPU needed). */

/* Sizes of the index and of the pooled statistics: rows = Hkv * NBq_tot,
 * max_nnz = Hkv * sum_r sum_{i < NBq_r} (off_r / B + i + 1) (every causal pair),
 * num_q_blocks = NBq_tot (rows of q_bar per head), num_k_blocks = NBk_tot (rows
 * of k_bar and v_bar per head). Any output pointer may be NULL. */
fp_status fp_index_shape(const fp_problem* p, int64_t* num_rows, int64_t* max_nnz,
                         int64_t* num_q_blocks, int64_t* num_k_blocks);

/* Bytes of DEVICE workspace fp_select_blocks and fp_stage1 need for this
 * problem: a tile ticket and one 8-byte look-back word per selection tile (a
 * tile is a run of query blocks of one KV head and request, cut to about equal
 * causal area: 256 tiles, 2.3 KB, at 128K tokens with 8 KV heads). A problem
 * of few, long rows (a chunk of a long prompt) also splits each tile's key
 * blocks among several workgroups, which adds an arrival count per tile, the
 * parts' row maxima and the tiles' fp32 scores (about 4 bytes per causal
 * block pair of the call: 0.8 MB for a 2048-token chunk at 128K). */
fp_status fp_select_workspace_bytes(const fp_problem* p, size_t* bytes);

/* Bytes of DEVICE workspace fp_sparse_prefill (sparse = 1) or fp_dense_prefill
 * (sparse = 0) needs with these attention args (NULL: defaults, automatic
 * split): bf16 copies of k_bar and v_bar for the correction (sparse only), for
 * FP8 a bf16 copy of the V codes (exact; K is read as FP8), and with split-KV the parts'
 * fp32 outputs and log-sum-exps. 0 for an unsplit dense bf16 problem. */
fp_status fp_attn_workspace_bytes(const fp_problem* p, const fp_attn_args* attn, int32_t sparse,
                                  size_t* bytes);

/* The same sizes through one call: which_call FP_CALL_SELECT (fp_select_blocks
 * and fp_stage1: fp_select_workspace_bytes), FP_CALL_SPARSE (fp_sparse_prefill)
 * or FP_CALL_DENSE (fp_dense_prefill), the last two with the default attention
 * arguments (automatic split; fp_attn_workspace_bytes takes explicit ones).
 * Host only. Unknown which_call: FP_ERR_ARG. */
enum { FP_CALL_SELECT = 0, FP_CALL_SPARSE = 1, FP_CALL_DENSE = 2 };
fp_status fp_workspace_bytes(const fp_problem* p, int32_t which_call, size_t* bytes);

/* The split-KV part count the attention calls will use for these args
 * (resolves num_splits = 0). */
fp_status fp_attn_num_splits(const fp_problem* p, const fp_attn_args* attn, int32_t* splits);

/* Validate a problem and (optionally, may be NULL) selection/attention args
 * exactly as the compute calls do, without touching any device pointer. */
fp_status fp_validate(const fp_problem* p, const fp_select_args* sel, const fp_attn_args* attn);

/* Stage 1a: pooled statistics ([digest] Figure 3: PackGQA packing and
 * block-mean pooling; Figure 4: mean key/value of a block).
 *   q_bar[h, i] = mean over the G heads of group h and the n tokens of query block i,
 *   k_bar[h, J], v_bar[h, J] = mean over the n_J positions of key block J,
 * each as dequantised values for FP8, accumulated in fp32. Every key block of
 * the sequence so far is pooled (in chunked prefill the earlier chunks' blocks
 * too). q, k, v: DEVICE inputs in the layouts above (k, v are the page pools
 * when paged). q_bar: DEVICE fp32 [Hkv, NBq_tot, d] output; k_bar, v_bar:
 * DEVICE fp32 [Hkv, P, d] outputs (P = pooled_pitch). */
fp_status fp_pool_blocks(const fp_problem* p, const void* q, const void* k, const void* v,
                         float* q_bar, float* k_bar, float* v_bar, void* stream);

/* Stage 1a for one chunk of a chunked prefill: as fp_pool_blocks, but pools
 * only the key blocks the chunk adds, J >= off_r / B. The blocks before the
 * chunk are complete and their means do not change, so their k_bar / v_bar
 * rows are neither read nor written here: they must already hold the values
 * an earlier call wrote (typically the previous chunk's call on the same
 * buffers, with a pooled_pitch that fits the whole prompt). In a batch of
 * several requests their rows only stay in place from call to call when
 * pooled_row_off fixes each request's region (kblk_off[r] moves as earlier
 * requests gain blocks). The pages note
 * that per-chunk selection repeats Stage 1 for every chunk ([podcast]);
 * this call keeps that repeated work proportional to the chunk. With
 * off_r = 0 it equals fp_pool_blocks. */
fp_status fp_pool_chunk_blocks(const fp_problem* p, const void* q, const void* k, const void* v,
                               float* q_bar, float* k_bar, float* v_bar, void* stream);

/* Stage 1b: scoring, threshold and CSR build ([digest] abstract; Table 7).
 * q_bar, k_bar: DEVICE outputs of fp_pool_blocks. row_ptr: DEVICE int32
 * [rows+1] output; row_ptr[rows] = nnz. col_idx: DEVICE int32 output with
 * room for col_capacity entries; col_capacity must be >= max_nnz of
 * fp_index_shape (checked before launch, so the kernels cannot overflow).
 * workspace: DEVICE scratch of at least fp_select_workspace_bytes bytes; its
 * contents on entry do not matter and are garbage on exit; calls that share a
 * workspace must not overlap. Scores are fp32 sums over the head dim in a
 * fixed order, decisions (z_J - max) >= ln(alpha) in fp32, the same whatever
 * the launch (chunked calls select exactly like a whole prefill). No score
 * is written to memory, except within the workspace when a problem of few,
 * long rows splits its tiles' key blocks. Two kernels: a small reset of the
 * workspace, then the fused score / threshold / prefix / compaction kernel.
 * Requests of more than FP_MAX_BLOCKS_PER_SEQ key blocks are rejected
 * (FP_ERR_UNSUPPORTED) by every call. */
fp_status fp_select_blocks(const fp_problem* p, const fp_select_args* sel, const float* q_bar,
                           const float* k_bar, int32_t* row_ptr, int32_t* col_idx,
                           int64_t col_capacity, void* workspace, size_t workspace_bytes,
                           void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * selection as fp_select_blocks, with its workspace in a fixed device array of
 * the library instead of a caller buffer. The caller passes only inputs and
 * outputs; the call allocates and frees nothing. The array holds the
 * workspace of problems up to FP_NOALLOC_MAX_SELECT_TILES selection tiles
 * (tiles as for fp_select_workspace_bytes, never split among workgroups here:
 * 256 tiles at 128K tokens with 8 KV heads, at least one per request and KV
 * head); larger problems return FP_ERR_CAPACITY before anything is enqueued.
 * Each GPU has one copy of the array, kept until the process ends, and every
 * call on that GPU uses it: calls that overlap on one GPU (other streams,
 * other threads) race and must not be made. The call uses the device current
 * on the calling thread. */
#define FP_NOALLOC_MAX_SELECT_TILES 65536
fp_status fp_select_blocks_noalloc(const fp_problem* p, const fp_select_args* sel, const float* q_bar,
                                   const float* k_bar, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                   void* stream);

/* Stage 1 in two kernels ([digest] Figure 3: PackGQA pooling and the CSR
 * index of selected blocks produced in one fused pass): fp_pool_blocks
 * (chunk_only = 0) or fp_pool_chunk_blocks (chunk_only = 1), whose kernel also
 * resets the selection workspace, then the selection kernel of
 * fp_select_blocks. Arguments, outputs and errors as in those two calls; every
 * argument of both is validated before either kernel is enqueued. */
fp_status fp_stage1(const fp_problem* p, const fp_select_args* sel, int32_t chunk_only, const void* q,
                    const void* k, const void* v, float* q_bar, float* k_bar, float* v_bar, int32_t* row_ptr,
                    int32_t* col_idx, int64_t col_capacity, void* workspace, size_t workspace_bytes, void* stream);

/* Stage 2: block-sparse attention with the fused mean correction ([digest]
 * Figure 3 Stage 2: exact path over CSR blocks and correction path merged in
 * one online softmax; Figure 4 surrogate |B_J| exp(s_J) (v_bar_J, 1)).
 * k_bar, v_bar: DEVICE fp32 from fp_pool_blocks (read only when
 * mean_correction = 1). row_ptr, col_idx: DEVICE CSR from fp_select_blocks
 * (or any CSR of the same shape with the diagonal in every row).
 * out: DEVICE bf16 [Tq, Hq, d]. lse: DEVICE fp32 [Hq, Tq], or NULL to skip.
 * workspace: DEVICE scratch of at least fp_attn_workspace_bytes(p, attn, 1) bytes
 * (may be NULL when that is 0); contents on entry do not matter, garbage on
 * exit; the call must not overlap another call using the same workspace. */
fp_status fp_sparse_prefill(const fp_problem* p, const fp_attn_args* attn, const void* q,
                            const void* k, const void* v, const float* k_bar, const float* v_bar,
                            const int32_t* row_ptr, const int32_t* col_idx, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Dense causal attention over every key at or before each query (the comparator
 * for the sparse path; mean_correction is ignored). Same layouts as above;
 * workspace as above with fp_attn_workspace_bytes(p, attn, 0). */
fp_status fp_dense_prefill(const fp_problem* p, const fp_attn_args* attn, const void* q,
                           const void* k, const void* v, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Device check of the inputs that fp_sparse_prefill trusts: the CSR of
 * selected blocks per KV head ([digest] Table 7; Figure 3, Stage 1 output)
 * and, for paged K / V, the page table ([digest] "What they did", Fix 3).
 * The prefill reads them without checks (none would be free at its rate);
 * a caller that builds its own CSR or page table can run this first.
 * row_ptr, col_idx: DEVICE CSR as for fp_sparse_prefill, col_idx holding
 * col_capacity entries (both NULL: check the page table only). err: DEVICE
 * int32, set to 0 and then to the OR of the FP_CHECK_* bits of every
 * problem found, in stream order (read it after the stream reaches this
 * point). Every read is bounded by the problem's sizes and col_capacity, so
 * a malformed index cannot make the check itself read out of range. */
enum {
  FP_CHECK_ROWPTR = 1,  /* row_ptr[0] != 0, an entry below its predecessor or past col_capacity */
  FP_CHECK_ORDER = 2,   /* a row's columns not strictly ascending                              */
  FP_CHECK_RANGE = 4,   /* a column outside [0, I] (I: the row's own key block)                */
  FP_CHECK_DIAG = 8,    /* a row with no columns, or whose last column is not I                */
  FP_CHECK_PAGE = 16    /* paged: a page id outside [0, num_pages) among the pages in use     */
};
fp_status fp_check_index(const fp_problem* p, const int32_t* row_ptr, const int32_t* col_idx,
                         int64_t col_capacity, int32_t* err, void* stream);

/* Static text for a status code; never NULL. */
const char* fp_status_string(fp_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* fp_last_error(void);

/* FPV2_ABI_VERSION of the built library. */
int32_t fp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FPV2_H */
