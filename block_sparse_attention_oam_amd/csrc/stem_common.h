// Shared device-side definitions of the Stem prefill library (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/stem.h"

#if !defined(__gfx950__) && defined(__HIP_DEVICE_COMPILE__)
#error "this library is written for gfx950 (MI355X) only"
#endif

namespace stem {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

// Per-request tables, passed by value in kernel arguments so lookups are scalar loads of the kernarg
// segment.  cu_blocks[r] = number of blocks in requests 0..r-1.
struct ReqTable {
  int32_t num_reqs;
  int32_t cu_seqlens[STEM_MAX_REQS + 1];
  int32_t cu_blocks[STEM_MAX_REQS + 1];
};

// Request that owns global block ib (binary search over cu_blocks; uniform across the workgroup).
__device__ __forceinline__ int find_request(const ReqTable& rt, int ib) {
  int lo = 0, hi = rt.num_reqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (rt.cu_blocks[mid] <= ib) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Two floats -> two bf16 (round to nearest even) packed in one dword, low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Four OCP e4m3fn codes (one dword) -> four floats, using the hardware fp8 conversion.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o[0] = lo[0];
  o[1] = lo[1];
  o[2] = hi[0];
  o[3] = hi[1];
}

// Address of token t (request-relative) of KV head g in a contiguous or paged K/V pool, in elements.
struct KvAddr {
  int32_t paged;
  int32_t page_size;
  int32_t pt_stride;
  const int32_t* page_table;
  int32_t hkv, d;

  __device__ __forceinline__ int64_t row(int r, int tok_base, int t, int g) const {
    if (!paged) return ((int64_t)(tok_base + t) * hkv + g) * d;
    const int page = page_table[(int64_t)r * pt_stride + t / page_size];
    return (((int64_t)page * page_size + (t % page_size)) * hkv + g) * d;
  }
};

}  // namespace stem
