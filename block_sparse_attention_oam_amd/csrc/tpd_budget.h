// Token Position Decay budgets in exact 64-bit integer arithmetic, usable on host and device.
//
// Source: "从Stem稀疏注意力看大模型推理的架构取舍", section "TPD：优先级排序": each query position gets a
// top-k budget that decays linearly from k_start at the start to k_end = mu * k_start at the end, and the
// total equals that of the uniform allocation (it is redistributed).  Section "HPC-Stem" fuses this "one
// formula per position" with the selection.
//
// Definition used (rows are query blocks i = 0..n-1 of one request):
//   C = n(n+1)/2,  T = clamp(floor(rho*C + 1/2), n, C)
//   w_i = 1 - (1-mu) i/(n-1);   r_i(x) = min(max(x w_i, 1), i+1);   x solves sum_i r_i(x) = T
//   P_i = r_0 + ... + r_i,  K_i = floor(P_i + 1/2),  k_i = K_i - K_{i-1}   (K_{-1} = 0)
//
// With mu = a/b, scale the weights to integers W_i = D - E i, D = b(n-1), E = b - a, and y = x / D so that
// r_i = min(max(y W_i, 1), i+1).  Rows that are capped at i+1 form a prefix [0, p), rows floored at 1 form
// a suffix [q, n), and the rows in between are linear: r_i = T' W_i / SW with T' = T - p(p+1)/2 - (n-q)
// and SW = W_p + ... + W_{q-1}.  p and q come from monotone predicates on the breakpoints
// (row i capped  <=>  F(c_i) <= T,  row m floored  <=>  F(f_m) >= T, c_i = (i+1)/W_i, f_m = 1/W_m, F the
// row sum), each a closed form, found by binary search.  Every quantity is an integer, so the device
// reproduces the exact rational budgets bit for bit.  Magnitudes stay below b * n^4, which the host
// checks against 2^62 before launching.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define TPD_HD __host__ __device__ inline
#else
#define TPD_HD inline
#endif

struct TpdPlan {
  int32_t n;      // blocks
  int32_t p, q;   // capped rows [0, p), linear rows [p, q), floored rows [q, n)
  int64_t T;      // total budget
  int64_t D, E;   // W_i = D - E i
  int64_t Tp;     // budget carried by the linear rows
  int64_t SW;     // sum of W over the linear rows
};

TPD_HD int64_t tpd_gcd(int64_t a, int64_t b) {
  while (b) {
    int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// Branch-free 64-bit min / max (|a - b| < 2^62 here).  Index comparisons elsewhere use 32-bit ints: on
// gfx950 a uniform signed 64-bit compare is a vector compare, and a scalar select fed by one has been seen
// to read a stale condition, so no 64-bit compare decides a select in this file.
TPD_HD int64_t tpd_max(int64_t a, int64_t b) {
  const int64_t d = b - a;
  return b - (d & (d >> 63));
}
TPD_HD int64_t tpd_min(int64_t a, int64_t b) {
  const int64_t d = b - a;
  return a + (d & (d >> 63));
}

// a <= b, from the sign of b - a (no relational 64-bit compare)
TPD_HD bool tpd_le(int64_t a, int64_t b) { return ((uint64_t)(b - a) >> 63) == 0; }

// floor(num / den) for den > 0
TPD_HD int64_t tpd_floordiv(int64_t num, int64_t den) {
  const int64_t q = num / den;
  const int64_t r = num - q * den;
  return q - (int64_t)(((uint64_t)num >> 63) & (uint64_t)(r != 0));
}

TPD_HD int64_t tpd_total(int32_t n, int64_t rho_num, int64_t rho_den) {
  const int64_t C = (int64_t)n * (n + 1) / 2;
  const int64_t T = tpd_floordiv(2 * rho_num * C + rho_den, 2 * rho_den);
  return tpd_min(tpd_max(T, n), C);
}

// sum_{i=a}^{b-1} (D - E i) for a <= b; (a+b-1)(b-a) is always even
TPD_HD int64_t tpd_sw(int64_t D, int64_t E, int32_t a, int32_t b) {
  const int64_t len = (int64_t)(b > a ? b - a : 0);
  return len * D - E * (((int64_t)a + b - 1) * len / 2);
}

// Is row i capped at the solution?  (F(c_i) <= T)
// Every weight W_i is positive because mu > 0 (W_{n-1} = a(n-1)).
TPD_HD bool tpd_capped(const TpdPlan& s, int32_t i) {
  const int64_t Wi = s.D - s.E * i;
  // rows floored at y = c_i: first m >= i+1 with (i+1) W_m <= W_i
  int32_t qf;
  if (s.E == 0) {
    qf = (i == 0) ? 1 : s.n;
  } else {
    const int64_t num = (int64_t)(i + 1) * s.D - Wi;  // m >= num / ((i+1) E)
    const int64_t den = (int64_t)(i + 1) * s.E;
    const int64_t c = -tpd_floordiv(-num, den);        // ceil
    qf = (int32_t)tpd_min(tpd_max(c, i + 1), s.n);
  }
  const int64_t lhs = (int64_t)(i + 1) * tpd_sw(s.D, s.E, i + 1, qf);
  const int64_t rhs = (s.T - (int64_t)(i + 1) * (i + 2) / 2 - (s.n - qf)) * Wi;
  return tpd_le(lhs, rhs);
}

// Is row m floored at the solution?  (F(f_m) >= T)
TPD_HD bool tpd_floored(const TpdPlan& s, int32_t m) {
  const int64_t Wm = s.D - s.E * m;
  if (s.E == 0) return tpd_le(s.T, s.n);  // all weights equal: at y = 1/D every row is 1
  // rows capped at y = f_m: i <= (D - W_m) / (E + W_m)
  const int64_t c = tpd_floordiv(s.D - Wm, s.E + Wm) + 1;
  const int32_t pc = (int32_t)tpd_max(tpd_min(c, m), 0);
  const int64_t lhs = ((int64_t)pc * (pc + 1) / 2 + s.n - m - s.T) * Wm + tpd_sw(s.D, s.E, pc, m);
  return tpd_le(0, lhs);
}

// Fields that depend only on (n, rho, mu).  Requires 0 < mu_num <= mu_den and 0 <= rho_num <= rho_den.
TPD_HD TpdPlan tpd_plan_init(int32_t n, int64_t rho_num, int64_t rho_den, int64_t mu_num, int64_t mu_den) {
  TpdPlan s;
  s.n = n;
  s.p = 0;
  s.q = n;
  s.T = tpd_total(n, rho_num, rho_den);
  const int64_t g = tpd_gcd(mu_num, mu_den);
  const int64_t a = mu_num / g, b = mu_den / g;
  s.D = b * (n > 1 ? n - 1 : 1);
  s.E = (n > 1) ? (b - a) : 0;
  s.Tp = 0;
  s.SW = 0;
  return s;
}

// Fields derived from the capped / floored row counts.
TPD_HD void tpd_plan_finish(TpdPlan& s, int32_t p, int32_t q) {
  s.p = p;
  s.q = q < p ? p : q;  // row 0 can be both capped and floored (value 1)
  s.Tp = s.T - (int64_t)s.p * (s.p + 1) / 2 - (s.n - s.q);
  s.SW = tpd_sw(s.D, s.E, s.p, s.q);
}

// Sequential solve (host helper; the kernel solves the same predicates with a wave-parallel search).
TPD_HD TpdPlan tpd_plan(int32_t n, int64_t rho_num, int64_t rho_den, int64_t mu_num, int64_t mu_den) {
  TpdPlan s = tpd_plan_init(n, rho_num, rho_den, mu_num, mu_den);
  // p = number of capped rows: the predicate holds on a prefix
  int32_t lo = 0, hi = n;  // answer in [lo, hi]
  while (lo < hi) {
    const int32_t mid = (lo + hi) / 2;
    if (tpd_capped(s, mid)) lo = mid + 1;
    else hi = mid;
  }
  const int32_t p = lo;
  // q = first floored row: the predicate holds on a suffix
  lo = 0;
  hi = n;
  while (lo < hi) {
    const int32_t mid = (lo + hi) / 2;
    if (tpd_floored(s, mid)) hi = mid;
    else lo = mid + 1;
  }
  tpd_plan_finish(s, p, lo);
  return s;
}

// K_i = floor(P_i + 1/2), the rounded prefix sum of the real budgets up to row i (K_{-1} = 0).
TPD_HD int64_t tpd_prefix(const TpdPlan& s, int32_t i) {
  if (i < 0) return 0;
  if (i < s.p) return (int64_t)(i + 1) * (i + 2) / 2;
  const int64_t cap = (int64_t)s.p * (s.p + 1) / 2;
  if (i < s.q) {
    const int64_t part = tpd_sw(s.D, s.E, s.p, i + 1);
    return cap + tpd_floordiv(2 * s.Tp * part + s.SW, 2 * s.SW);
  }
  return cap + s.Tp + (i + 1 - s.q);
}

TPD_HD int64_t tpd_row_budget(const TpdPlan& s, int32_t i) { return tpd_prefix(s, i) - tpd_prefix(s, i - 1); }
