// Device check of a CSR index and a page table before they are handed to the
// attention kernel, which reads both without checks.
//
// Method: "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context LLM
// Serving" (metallab.ai paper digest), Table 7 (a CSR of the selected blocks
// per KV head) and "What they did", Fix 3 (paged KV cache).
//
// One wave per CSR row: the row's extent is checked against its neighbour
// and the column capacity before any column is read, then lanes read the
// columns (each with its predecessor) and test order, range and the closing
// diagonal. Workgroups past the rows check one request's page ids each.
// Findings are OR-ed into one word.
#include "common.h"
#include "launch.h"

namespace fpv2 {

namespace {

constexpr int kCheckThreads = 256;
constexpr int kRowsPerWG = kCheckThreads / 64;

__global__ void check_clear_kernel(int32_t* err) { *err = 0; }

__global__ __launch_bounds__(kCheckThreads) void check_kernel(CheckParams p) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row_wgs = p.row_ptr ? (p.rows + kRowsPerWG - 1) / kRowsPerWG : 0;
  int flags = 0;
  if ((int)blockIdx.x < row_wgs) {
    const int g = (int)blockIdx.x * kRowsPerWG + w;
    if (g < p.rows) {
      const int b = g % p.NBq_tot;
      int r = 0;
      while (r + 1 < p.rt.R && p.rt.blk_off[r + 1] <= b) ++r;
      const int I = p.rt.qb0[r] + (b - p.rt.blk_off[r]);
      const int rp0 = p.row_ptr[g], rp1 = p.row_ptr[g + 1];
      if (g == 0 && rp0 != 0) flags |= FP_CHECK_ROWPTR;
      if (rp0 < 0 || rp1 < rp0 || (int64_t)rp1 > p.cap) {
        flags |= FP_CHECK_ROWPTR;
      } else if (rp1 == rp0) {
        flags |= FP_CHECK_DIAG;
      } else {
        const int n = rp1 - rp0;
        for (int k = lane; k < n; k += 64) {
          const int c = p.col_idx[rp0 + k];
          if (k > 0 && c <= p.col_idx[rp0 + k - 1]) flags |= FP_CHECK_ORDER;
          if (c < 0 || c > I) flags |= FP_CHECK_RANGE;
          if (k == n - 1 && c != I) flags |= FP_CHECK_DIAG;
        }
      }
    }
  } else if (p.kv.paged) {
    const int r = (int)blockIdx.x - row_wgs;
    if (r < p.rt.R) {
      const int Lk = p.rt.ktok_off[r + 1] - p.rt.ktok_off[r];
      const int npages = (Lk + p.kv.page_size - 1) / p.kv.page_size;  // <= max_pages (host-checked)
      const int32_t* pt = p.kv.page_table + (int64_t)r * p.kv.max_pages;
      for (int j = threadIdx.x; j < npages; j += kCheckThreads) {
        const int id = pt[j];
        if (id < 0 || id >= p.num_pages) flags |= FP_CHECK_PAGE;
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) flags |= __shfl_xor(flags, o);
  if (lane == 0 && flags) atomicOr(p.err, flags);
}

}  // namespace

hipError_t launch_check(const CheckParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(check_clear_kernel, dim3(1), dim3(1), 0, stream, p.err);
  const int row_wgs = p.row_ptr ? (p.rows + kRowsPerWG - 1) / kRowsPerWG : 0;
  const int wgs = row_wgs + (p.kv.paged ? p.rt.R : 0);
  if (wgs > 0) hipLaunchKernelGGL(check_kernel, dim3(wgs), dim3(kCheckThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fpv2
