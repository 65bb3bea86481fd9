// Device helpers shared by the selection kernels (tpd_topk.hip, score_topk.hip): the per-wave TPD budget
// plan and the per-row top-k on order-preserving keys.
//
// Source: "从Stem稀疏注意力看大模型推理的架构取舍", sections "TPD：优先级排序" and "HPC-Stem：评估选块，快几十倍".
#pragma once

#include "stem_internal.h"
#include "tpd_budget.h"

namespace stem {

// Order-preserving map float -> uint32 (larger float, larger key); -0 is folded onto +0.
__device__ __forceinline__ uint32_t ord_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of leading indices in [0, n) where pred holds (pred true on a prefix), via 64-ary search.
// Indices are 32-bit (see the note on 64-bit compares in tpd_budget.h).
template <typename Pred>
__device__ __forceinline__ int32_t wave_prefix_count(int32_t n, int lane, Pred pred) {
  int32_t lo = 0, hi = n;
  while (lo < hi) {
    const int32_t step = (hi - lo + 63) >> 6;
    const int32_t x = lo + lane * step;
    const bool t = (x < hi) && pred(x);
    const int c = __popcll(__ballot(t));
    if (c == 0) {
      hi = lo;
    } else {
      lo = lo + (c - 1) * step + 1;
      hi = min(hi, lo - 1 + step);
    }
  }
  return lo;
}

// The budget plan of a request with n blocks, solved by one wavefront.
__device__ __forceinline__ TpdPlan wave_plan(int32_t n, int32_t rho_num, int32_t rho_den, int32_t mu_num,
                                             int32_t mu_den, int lane) {
  TpdPlan s = tpd_plan_init(n, rho_num, rho_den, mu_num, mu_den);
  const int32_t p = wave_prefix_count(n, lane, [&](int32_t i) { return tpd_capped(s, i); });
  const int32_t q = wave_prefix_count(n, lane, [&](int32_t m) { return !tpd_floored(s, m); });
  tpd_plan_finish(s, p, q);
  return s;
}

// Top-k of one row held by one wavefront: key[s] is the key of block j = lane + 64 s (0 for j > i or
// past the row).  Selects the k largest keys, equal keys in increasing j; writes the row's mask words
// (all mask_words of them, zero past the row) and returns nothing else.
template <int NS>
__device__ __forceinline__ void select_row(const uint32_t (&key)[NS], int nslot, int k, int lane,
                                           uint32_t* mrow, int mask_words) {
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // k-th largest key: the largest tau with #{key >= tau} >= k (valid keys are >= 0x007FFFFF > 0, invalid
  // ones 0).  All valid keys share the bits above the highest bit where the row's largest and smallest
  // valid keys differ, so tau does too: the bit-by-bit search starts below that common prefix.  It stops
  // as soon as exactly k keys reach the candidate (those are then the k largest, with no tie at the
  // boundary), which gives the same selection as running it to the last bit.
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < nslot && key[s] != 0u) {
      kmax = max(kmax, key[s]);
      kmin = min(kmin, key[s]);
    }
  for (int o = 1; o < 64; o <<= 1) {
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
  }
  const uint32_t diff = kmax ^ kmin;
  const int top = diff == 0u ? -1 : 31 - __clz(diff);  // highest differing bit (-1: all keys equal)
  uint32_t tau;                                          // the common prefix, lower bits clear
  if (top < 0) tau = kmax;
  else if (top == 31) tau = 0u;
  else tau = kmax & ~((2u << top) - 1u);
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (s < nslot) cnt += __popcll(__ballot(key[s] >= cand));
    if (cnt >= k) tau = cand;
    if (cnt == k) break;
  }
  int gt = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < nslot) gt += __popcll(__ballot(key[s] > tau));
  const int need = k - gt;
  int taken = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s < nslot) {
      const uint64_t eq = __ballot(key[s] == tau);
      const int rank = taken + __popcll(eq & below);
      const bool sel = key[s] > tau || (key[s] == tau && rank < need);
      const uint64_t selm = __ballot(sel);
      taken += __popcll(eq);
      if (lane < 2 && 2 * s + lane < mask_words)
        mrow[2 * s + lane] = lane == 0 ? (uint32_t)selm : (uint32_t)(selm >> 32);
    }
  }
  for (int w = 2 * nslot + lane; w < mask_words; w += 64) mrow[w] = 0u;
}

}  // namespace stem
