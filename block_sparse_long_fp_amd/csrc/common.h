// Shared device-side definitions of the gfx950 block-sparse prefill kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fpv2.h"

namespace fpv2 {

constexpr int kHeadDim = FP_HEAD_DIM;   // d
constexpr int kMaxSeqs = FP_MAX_SEQS;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Ragged batch description, passed by value as a kernel argument. Built on the
// host from the host-side cu_seqlens / cu_seqlens_k, so no device lookup table
// is needed. Request r has Lk keys (positions 0 .. Lk-1) and its last Lq
// positions as queries; qb0 = (Lk - Lq) / B is the key block of its first
// query block (0 for a whole prefill).
struct ReqTable {
  int32_t R;                         // requests
  int32_t nb_max;                    // max_r NBk_r
  int32_t tok_off[kMaxSeqs + 1];     // query tokens: cu_seqlens
  int32_t ktok_off[kMaxSeqs + 1];    // key tokens: cu_seqlens_k
  int32_t blk_off[kMaxSeqs + 1];     // prefix sums of NBq_r (q_bar and CSR rows)
  int32_t kblk_off[kMaxSeqs + 1];    // prefix sums of NBk_r (k_bar and v_bar rows)
  int32_t qb0[kMaxSeqs];             // first query block's key-block id
  int32_t prow_off[kMaxSeqs];        // first k_bar / v_bar row (per KV head) of each request
};

// K/V addressing: contiguous [T, Hkv, d] or paged [pages, page_size, Hkv, d].
struct KVAddr {
  const int32_t* page_table;  // [R, max_pages] (paged only)
  int32_t page_size;
  int32_t max_pages;
  int32_t paged;
};

// Element offset of (request r, key position t, kv head h, dim 0).
__device__ __forceinline__ int64_t kv_elem_offset(const KVAddr& a, const ReqTable& rt, int r, int t, int h,
                                                  int Hkv) {
  int64_t row;
  if (a.paged) {
    const int page = a.page_table[(int64_t)r * a.max_pages + t / a.page_size];
    row = (int64_t)page * a.page_size + (t % a.page_size);
  } else {
    row = (int64_t)rt.ktok_off[r] + t;
  }
  return (row * Hkv + h) * kHeadDim;
}

// FP8 inputs are OCP E4M3 (FN) codes, the encoding the gfx950 conversion
// and matrix instructions take (v_cvt_scalef32_pk_*_fp8 with scale 1 widen
// them exactly).

// bf16 <-> float helpers on raw bits.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// Loads through explicitly global / LDS pointers. Pointers merged from
// several sources otherwise become generic (flat) accesses, which count
// against both the vector-memory and the LDS wait counters and so force a
// wait for outstanding global loads before every LDS read.
typedef const __attribute__((address_space(1))) u32x4 g_u32x4;
typedef const __attribute__((address_space(1))) int32_t g_int32;
typedef const __attribute__((address_space(1))) uint8_t g_uint8;
typedef const __attribute__((address_space(1))) float g_float;
typedef const __attribute__((address_space(3))) int32_t l_int32;
// Constant address space: memory no thread writes while the kernel runs.
// Wave-uniform loads through it become scalar loads (s_load).
typedef const __attribute__((address_space(4))) int32_t c_int32;
__device__ __forceinline__ int32_t sload_i32(const int32_t* p) { return *(c_int32*)(p); }
__device__ __forceinline__ uint4 gload16(g_u32x4* p) { return __builtin_bit_cast(uint4, *p); }
__device__ __forceinline__ int32_t gload_i32(const int32_t* p) { return *(g_int32*)(p); }
__device__ __forceinline__ int32_t lload_i32(const int32_t* p) { return *(l_int32*)(p); }

}  // namespace fpv2
