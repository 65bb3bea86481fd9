// Host side of the C ABI declared in include/stem.h: argument validation (before any HIP call),
// workspace layout, per-request tables, the gfx950 device check, and the kernel launches.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "stem_internal.h"

using namespace stem;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return STEM_OK;
}

// Validate the descriptor and derive the plan (request tables, block counts).  Pure host code.
int make_plan(const stem_problem* p, Plan* plan) {
  if (!p) return fail(STEM_E_INVALID_ARG, "problem descriptor is NULL");
  if (p->num_reqs < 1 || p->num_reqs > STEM_MAX_REQS)
    return fail(STEM_E_INVALID_ARG, "num_reqs = %d, must be in [1, %d]", p->num_reqs, STEM_MAX_REQS);
  if (!p->cu_seqlens) return fail(STEM_E_INVALID_ARG, "cu_seqlens is NULL");
  if (p->cu_seqlens[0] != 0) return fail(STEM_E_INVALID_ARG, "cu_seqlens[0] = %d, must be 0", p->cu_seqlens[0]);
  if (p->hq < 1 || p->hkv < 1 || p->hq % p->hkv != 0)
    return fail(STEM_E_INVALID_ARG, "hq = %d, hkv = %d: both must be >= 1 and hq %% hkv == 0", p->hq, p->hkv);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(STEM_E_UNSUPPORTED, "head_dim = %d, supported: 64, 128", p->head_dim);
  if (p->block != 64 && p->block != 128) return fail(STEM_E_UNSUPPORTED, "block = %d, supported: 64, 128", p->block);
  if (p->dtype != STEM_F32 && p->dtype != STEM_BF16 && p->dtype != STEM_FP8_E4M3)
    return fail(STEM_E_INVALID_ARG, "dtype = %d is not a stem_dtype", p->dtype);
  if (p->dtype == STEM_FP8_E4M3 && (!p->q_scale || !p->k_scale || !p->v_scale))
    return fail(STEM_E_INVALID_ARG, "fp8 inputs need q_scale, k_scale and v_scale");
  plan->p = p;
  plan->rt.num_reqs = p->num_reqs;
  plan->rt.cu_seqlens[0] = 0;
  plan->rt.cu_blocks[0] = 0;
  int64_t nb = 0;
  int32_t max_n = 0, max_len = 0;
  for (int r = 0; r < p->num_reqs; ++r) {
    const int64_t len = (int64_t)p->cu_seqlens[r + 1] - p->cu_seqlens[r];
    if (len < 0) return fail(STEM_E_INVALID_ARG, "cu_seqlens decreases at request %d", r);
    const int64_t n = (len + p->block - 1) / p->block;
    nb += n;
    if (n > max_n) max_n = (int32_t)n;
    if (len > max_len) max_len = (int32_t)len;
    plan->rt.cu_seqlens[r + 1] = p->cu_seqlens[r + 1];
    plan->rt.cu_blocks[r + 1] = (int32_t)nb;
  }
  if (nb == 0) return fail(STEM_E_INVALID_ARG, "all requests are empty");
  if (nb * (int64_t)p->hq >= ((int64_t)1 << 31)) return fail(STEM_E_UNSUPPORTED, "hq * blocks exceeds 2^31");
  plan->NB = nb;
  plan->max_n = max_n;
  plan->max_len = max_len;
  plan->tokens = p->cu_seqlens[p->num_reqs];
  KvAddr& kv = plan->kv;
  kv.paged = p->kv_paged ? 1 : 0;
  kv.hkv = p->hkv;
  kv.d = p->head_dim;
  kv.page_size = 1;
  kv.pt_stride = 0;
  kv.page_table = nullptr;
  if (p->kv_paged) {
    if (p->page_size < 16 || p->page_size % 16 != 0)
      return fail(STEM_E_INVALID_ARG, "page_size = %d, must be a positive multiple of 16", p->page_size);
    if (!p->page_table) return fail(STEM_E_INVALID_ARG, "paged K/V without a page table");
    if (p->num_pages < 1) return fail(STEM_E_INVALID_ARG, "num_pages = %d", p->num_pages);
    const int64_t need = ((int64_t)max_len + p->page_size - 1) / p->page_size;
    if (p->page_table_stride < need)
      return fail(STEM_E_INVALID_ARG, "page_table_stride = %d < %lld pages of the longest request",
                  p->page_table_stride, (long long)need);
    kv.page_size = p->page_size;
    kv.pt_stride = p->page_table_stride;
    kv.page_table = p->page_table;
  }
  return STEM_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

void layout(const Plan& pl, size_t* oq, size_t* ok_, size_t* om, size_t* total) {
  const stem_problem* p = pl.p;
  const size_t qb = (size_t)p->hq * pl.NB * p->head_dim * sizeof(float);
  const size_t kb = (size_t)p->hkv * pl.NB * p->head_dim * sizeof(float);
  const size_t mb = (size_t)p->hkv * pl.NB * sizeof(float);
  *oq = 0;
  *ok_ = align256(qb);
  *om = *ok_ + align256(kb);
  *total = *om + align256(mb);
}

// gfx950 check of the current device, cached per device id.
int check_device() {
  static std::mutex mu;
  static std::vector<int> state;  // 0 unknown, 1 ok, 2 bad
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(STEM_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  if ((int)state.size() <= dev) state.resize(dev + 1, 0);
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(STEM_E_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    state[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    if (state[dev] == 2) return fail(STEM_E_UNSUPPORTED, "device %d is %s, this library runs on gfx950 only", dev,
                                     prop.gcnArchName);
  }
  if (state[dev] == 2) return fail(STEM_E_UNSUPPORTED, "device %d is not gfx950", dev);
  return STEM_OK;
}

// ---- static scratch of stem_score_noalloc: the pooled q-bar, k-bar and M of its calls live here instead of
// in a caller workspace.  One copy per device (the code object's global), held until the process ends.  In
// host code `scratch` is only a stand-in for the symbol: kernels get the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device and kept.
static __device__ __align__(256) uint8_t scratch[STEM_SCRATCH_BYTES];

int scratch_address(void** out) {
  static std::mutex mu;
  static std::vector<void*> addr;  // per device id; nullptr until looked up
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(STEM_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(STEM_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return STEM_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(STEM_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int check_rational(const char* name, int32_t num, int32_t den, bool allow_zero) {
  if (den <= 0) return fail(STEM_E_INVALID_ARG, "%s denominator %d must be > 0", name, den);
  if (num < (allow_zero ? 0 : 1) || num > den)
    return fail(STEM_E_INVALID_ARG, "%s = %d/%d must lie in %s, 1]", name, num, den, allow_zero ? "[0" : "(0");
  return STEM_OK;
}

// Every intermediate of the integer budget solve stays below mu_den * n^4 (and rho_den * n^2).
int check_budget_range(int64_t n, int32_t rho_den, int32_t mu_num, int32_t mu_den) {
  const int64_t g = tpd_gcd(mu_num, mu_den);
  const double b = (double)(mu_den / g);
  const double bound = 2.0 * b * (double)n * n * (double)n * n + (double)rho_den * n * n * 2.0;
  if (bound >= 4.0e18) return fail(STEM_E_UNSUPPORTED, "n = %lld blocks with mu denominator %d overflows the exact "
                                   "64-bit budget arithmetic", (long long)n, mu_den);
  return STEM_OK;
}

}  // namespace

extern "C" {

const char* stem_status_string(int status) {
  switch (status) {
    case STEM_OK: return "STEM_OK";
    case STEM_E_INVALID_ARG: return "STEM_E_INVALID_ARG";
    case STEM_E_UNSUPPORTED: return "STEM_E_UNSUPPORTED";
    case STEM_E_WORKSPACE: return "STEM_E_WORKSPACE";
    case STEM_E_HIP: return "STEM_E_HIP";
    default: return "unknown status";
  }
}

const char* stem_last_error(void) { return g_last_error.c_str(); }

int stem_block_counts(const stem_problem* p, int64_t* total_blocks, int32_t* max_blocks) {
  Plan pl;
  const int st = make_plan(p, &pl);
  if (st != STEM_OK) return st;
  if (total_blocks) *total_blocks = pl.NB;
  if (max_blocks) *max_blocks = pl.max_n;
  return ok();
}

size_t stem_workspace_bytes(const stem_problem* p) {
  Plan pl;
  if (make_plan(p, &pl) != STEM_OK) return 0;
  size_t a, b, c, t;
  layout(pl, &a, &b, &c, &t);
  ok();
  return t;
}

int stem_workspace_layout(const stem_problem* p, size_t* off_qbar, size_t* off_kbar, size_t* off_m) {
  Plan pl;
  const int st = make_plan(p, &pl);
  if (st != STEM_OK) return st;
  size_t a, b, c, t;
  layout(pl, &a, &b, &c, &t);
  if (off_qbar) *off_qbar = a;
  if (off_kbar) *off_kbar = b;
  if (off_m) *off_m = c;
  return ok();
}

int stem_tpd_budgets_host(int32_t n, int32_t rho_num, int32_t rho_den, int32_t mu_num, int32_t mu_den,
                          int32_t* k_out) {
  if (n < 1) return fail(STEM_E_INVALID_ARG, "n = %d must be >= 1", n);
  if (!k_out) return fail(STEM_E_INVALID_ARG, "k_out is NULL");
  int st = check_rational("rho", rho_num, rho_den, true);
  if (st != STEM_OK) return st;
  st = check_rational("mu", mu_num, mu_den, false);
  if (st != STEM_OK) return st;
  st = check_budget_range(n, rho_den, mu_num, mu_den);
  if (st != STEM_OK) return st;
  const TpdPlan s = tpd_plan(n, rho_num, rho_den, mu_num, mu_den);
  for (int32_t i = 0; i < n; ++i) k_out[i] = (int32_t)tpd_row_budget(s, i);
  return ok();
}

// Validation shared by the entry points that pool (stem_score, stem_score_select) and the pooling launch.
static int check_pool_args(const stem_problem* p, const Plan& pl, const void* q, const void* k, const void* v,
                           float beta, void* ws, size_t ws_bytes) {
  (void)p;
  if (!q || !k || !v) return fail(STEM_E_INVALID_ARG, "q, k and v must be non-NULL");
  if (!isfinite(beta)) return fail(STEM_E_INVALID_ARG, "beta is not finite");
  size_t oq, okk, om, need;
  layout(pl, &oq, &okk, &om, &need);
  if (!ws || ws_bytes < need)
    return fail(STEM_E_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : (size_t)0, need);
  if (((uintptr_t)ws & 255) != 0) return fail(STEM_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15)
    return fail(STEM_E_INVALID_ARG, "q, k and v must be 16-byte aligned");
  return STEM_OK;
}

static hipError_t launch_pooling(const stem_problem* p, const Plan& pl, const void* q, const void* k, const void* v,
                                 void* ws, hipStream_t s) {
  size_t oq, okk, om, need;
  layout(pl, &oq, &okk, &om, &need);
  PoolArgs pa;
  pa.q = q;
  pa.k = k;
  pa.v = v;
  pa.qbar = (float*)((char*)ws + oq);
  pa.kbar = (float*)((char*)ws + okk);
  pa.M = (float*)((char*)ws + om);
  pa.q_scale = p->q_scale;
  pa.k_scale = p->k_scale;
  pa.v_scale = p->v_scale;
  pa.hq = p->hq;
  pa.hkv = p->hkv;
  pa.d = p->head_dim;
  pa.B = p->block;
  pa.NB = pl.NB;
  const int eb = p->dtype == STEM_F32 ? 4 : (p->dtype == STEM_BF16 ? 2 : 1);
  const int epl = 16 / eb;
  pa.q_chunks = (p->hq * p->head_dim / epl + 255) / 256;
  pa.kv_chunks = (p->hkv * p->head_dim / epl + 255) / 256;
  pa.kv = pl.kv;
  pa.rt = pl.rt;
  return launch_pool(pa, p->dtype, s);
}

}  // extern "C"

// The launches of stem_score (pooling into ws, then the scoring GEMM), after validation.
static int launch_score_stage(const stem_problem* p, const Plan& pl, const void* q, const void* k, const void* v,
                              float beta, float* scores, int64_t score_row_stride, void* ws, hipStream_t s) {
  hipError_t e = launch_pooling(p, pl, q, k, v, ws, s);
  if (e != hipSuccess) return hip_status(e, "pool launch");
  size_t oq, okk, om, need;
  layout(pl, &oq, &okk, &om, &need);
  ScoreArgs sa;
  sa.qbar = (const float*)((char*)ws + oq);
  sa.kbar = (const float*)((char*)ws + okk);
  sa.M = (const float*)((char*)ws + om);
  sa.scores = scores;
  sa.stride = score_row_stride;
  sa.NB = pl.NB;
  sa.hq = p->hq;
  sa.hkv = p->hkv;
  sa.d = p->head_dim;
  sa.beta = beta;
  sa.inv_sqrt_d = 1.0f / sqrtf((float)p->head_dim);
  sa.rt = pl.rt;
  e = launch_score(sa, pl.max_n, p->num_reqs, s);
  return hip_status(e, "score launch");
}

extern "C" {

int stem_score(const stem_problem* p, const void* q, const void* k, const void* v, float beta, float* scores,
               int64_t score_row_stride, void* ws, size_t ws_bytes, void* stream) {
  Plan pl;
  int st = make_plan(p, &pl);
  if (st != STEM_OK) return st;
  if (!scores) return fail(STEM_E_INVALID_ARG, "q, k, v and scores must be non-NULL");
  if (score_row_stride < pl.max_n)
    return fail(STEM_E_INVALID_ARG, "score_row_stride = %lld < %d blocks of the longest request",
                (long long)score_row_stride, pl.max_n);
  st = check_pool_args(p, pl, q, k, v, beta, ws, ws_bytes);
  if (st != STEM_OK) return st;
  st = check_device();
  if (st != STEM_OK) return st;
  return launch_score_stage(p, pl, q, k, v, beta, scores, score_row_stride, ws, (hipStream_t)stream);
}

int stem_score_noalloc(const stem_problem* p, const void* q, const void* k, const void* v, float beta,
                       float* scores, int64_t score_row_stride, void* stream) {
  Plan pl;
  int st = make_plan(p, &pl);
  if (st != STEM_OK) return st;
  if (!scores) return fail(STEM_E_INVALID_ARG, "q, k, v and scores must be non-NULL");
  if (score_row_stride < pl.max_n)
    return fail(STEM_E_INVALID_ARG, "score_row_stride = %lld < %d blocks of the longest request",
                (long long)score_row_stride, pl.max_n);
  size_t oq, okk, om, need;
  layout(pl, &oq, &okk, &om, &need);
  if (need > (size_t)STEM_SCRATCH_BYTES)
    return fail(STEM_E_UNSUPPORTED, "this problem pools %zu bytes; the static scratch of stem_score_noalloc holds "
                "%zu (use stem_score with a workspace)", need, (size_t)STEM_SCRATCH_BYTES);
  // the scratch is 256-byte aligned and large enough: validate the rest as stem_score does
  st = check_pool_args(p, pl, q, k, v, beta, (void*)(uintptr_t)256, (size_t)STEM_SCRATCH_BYTES);
  if (st != STEM_OK) return st;
  st = check_device();
  if (st != STEM_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != STEM_OK) return st;
  return launch_score_stage(p, pl, q, k, v, beta, scores, score_row_stride, ws, (hipStream_t)stream);
}

int stem_quantize_fp8(const stem_problem* p, const void* q, const void* k, const void* v, void* q8, void* k8,
                      void* v8, float* q_scale, float* k_scale, float* v_scale, void* stream) {
  Plan pl;
  int st = make_plan(p, &pl);
  if (st != STEM_OK) return st;
  if (p->dtype != STEM_FP8_E4M3 || p->kv_paged)
    return fail(STEM_E_UNSUPPORTED, "quantisation describes an fp8 layer with contiguous K/V");
  if (!q || !k || !v || !q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale)
    return fail(STEM_E_INVALID_ARG, "q, k, v, q8, k8, v8 and the scale arrays must be non-NULL");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)q8 | (uintptr_t)k8 | (uintptr_t)v8) & 15)
    return fail(STEM_E_INVALID_ARG, "q, k, v, q8, k8 and v8 must be 16-byte aligned");
  st = check_device();
  if (st != STEM_OK) return st;
  PoolArgs pa;
  pa.q = q;
  pa.k = k;
  pa.v = v;
  pa.q8 = q8;
  pa.k8 = k8;
  pa.v8 = v8;
  pa.hq = p->hq;
  pa.hkv = p->hkv;
  pa.d = p->head_dim;
  pa.B = p->block;
  pa.NB = pl.NB;
  pa.kv = pl.kv;
  pa.rt = pl.rt;
  return hip_status(launch_quant(pa, q_scale, k_scale, v_scale, pl.tokens, (hipStream_t)stream), "quantise launch");
}

int stem_quantize_score(const stem_problem* p, const void* q, const void* k, const void* v, void* q8, void* k8,
                        void* v8, float* q_scale, float* k_scale, float* v_scale, float beta, float* scores,
                        int64_t score_row_stride, void* ws, size_t ws_bytes, void* stream) {
  Plan pl;
  int st = make_plan(p, &pl);
  if (st != STEM_OK) return st;
  if (p->dtype != STEM_FP8_E4M3 || p->kv_paged)
    return fail(STEM_E_UNSUPPORTED, "quantising scoring describes an fp8 layer with contiguous K/V");
  if (!q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale || !scores)
    return fail(STEM_E_INVALID_ARG, "q8, k8, v8, the scale arrays and scores must be non-NULL");
  if (score_row_stride < pl.max_n)
    return fail(STEM_E_INVALID_ARG, "score_row_stride = %lld < %d", (long long)score_row_stride, pl.max_n);
  st = check_pool_args(p, pl, q, k, v, beta, ws, ws_bytes);
  if (st != STEM_OK) return st;
  if (((uintptr_t)q8 | (uintptr_t)k8 | (uintptr_t)v8) & 15)
    return fail(STEM_E_INVALID_ARG, "q8, k8 and v8 must be 16-byte aligned");
  st = check_device();
  if (st != STEM_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  size_t oq, okk, om, need;
  layout(pl, &oq, &okk, &om, &need);
  PoolArgs pa;
  pa.q = q;
  pa.k = k;
  pa.v = v;
  pa.q8 = q8;
  pa.k8 = k8;
  pa.v8 = v8;
  pa.qbar = (float*)((char*)ws + oq);
  pa.kbar = (float*)((char*)ws + okk);
  pa.M = (float*)((char*)ws + om);
  pa.q_scale = q_scale;
  pa.k_scale = k_scale;
  pa.v_scale = v_scale;
  pa.hq = p->hq;
  pa.hkv = p->hkv;
  pa.d = p->head_dim;
  pa.B = p->block;
  pa.NB = pl.NB;
  pa.q_chunks = (p->hq * p->head_dim / 16 + 255) / 256;  // fp8 lane layout: 16 elements per lane
  pa.kv_chunks = (p->hkv * p->head_dim / 16 + 255) / 256;
  pa.kv = pl.kv;
  pa.rt = pl.rt;
  hipError_t e = launch_quant_pool(pa, q_scale, k_scale, v_scale, pl.tokens, s);
  if (e != hipSuccess) return hip_status(e, "quantising pool launch");
  ScoreArgs sa;
  sa.qbar = pa.qbar;
  sa.kbar = pa.kbar;
  sa.M = pa.M;
  sa.scores = scores;
  sa.stride = score_row_stride;
  sa.NB = pl.NB;
  sa.hq = p->hq;
  sa.hkv = p->hkv;
  sa.d = p->head_dim;
  sa.beta = beta;
  sa.inv_sqrt_d = 1.0f / sqrtf((float)p->head_dim);
  sa.rt = pl.rt;
  return hip_status(launch_score(sa, pl.max_n, p->num_reqs, s), "score launch");
}

// Budget and mask arguments shared by stem_tpd_topk and stem_score_select.
static int check_select_args(const Plan& pl, int32_t rho_num, int32_t rho_den, int32_t mu_num, int32_t mu_den,
                             const uint32_t* mask, int32_t mask_row_words, const int32_t* counts) {
  if (!mask || !counts) return fail(STEM_E_INVALID_ARG, "mask and counts must be non-NULL");
  if (mask_row_words < (pl.max_n + 31) / 32)
    return fail(STEM_E_INVALID_ARG, "mask_row_words = %d < %d", mask_row_words, (pl.max_n + 31) / 32);
  int st = check_rational("rho", rho_num, rho_den, true);
  if (st != STEM_OK) return st;
  st = check_rational("mu", mu_num, mu_den, false);
  if (st != STEM_OK) return st;
  return check_budget_range(pl.max_n, rho_den, mu_num, mu_den);
}

int stem_score_select(const stem_problem* p, const void* q, const void* k, const void* v, float beta,
                      int32_t rho_num, int32_t rho_den, int32_t mu_num, int32_t mu_den, uint32_t* mask,
                      int32_t mask_row_words, int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  Plan pl;
  int st = make_plan(p, &pl);
  if (st != STEM_OK) return st;
  st = check_pool_args(p, pl, q, k, v, beta, ws, ws_bytes);
  if (st != STEM_OK) return st;
  st = check_select_args(pl, rho_num, rho_den, mu_num, mu_den, mask, mask_row_words, counts);
  if (st != STEM_OK) return st;
  if (pl.max_n > 2048)
    return fail(STEM_E_UNSUPPORTED, "fused scoring and selection supports up to 2048 blocks per request");
  st = check_device();
  if (st != STEM_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_pooling(p, pl, q, k, v, ws, s);
  if (e != hipSuccess) return hip_status(e, "pool launch");
  size_t oq, okk, om, need;
  layout(pl, &oq, &okk, &om, &need);
  ScoreTopkArgs a{};
  a.qbar = (const float*)((char*)ws + oq);
  a.kbar = (const float*)((char*)ws + okk);
  a.M = (const float*)((char*)ws + om);
  a.mask = mask;
  a.mask_words = mask_row_words;
  a.counts = counts;
  a.NB = pl.NB;
  a.hq = p->hq;
  a.hkv = p->hkv;
  a.d = p->head_dim;
  a.beta = beta;
  a.inv_sqrt_d = 1.0f / sqrtf((float)p->head_dim);
  a.rho_num = rho_num;
  a.rho_den = rho_den;
  a.mu_num = mu_num;
  a.mu_den = mu_den;
  a.rt = pl.rt;
  return hip_status(launch_score_topk(a, pl.max_n, p->num_reqs, s), "score-select launch");
}

int stem_tpd_topk(const stem_problem* p, const float* scores, int64_t score_row_stride, int32_t rho_num,
                  int32_t rho_den, int32_t mu_num, int32_t mu_den, uint32_t* mask, int32_t mask_row_words,
                  int32_t* counts, void* stream) {
  Plan pl;
  int st = make_plan(p, &pl);
  if (st != STEM_OK) return st;
  if (!scores || !mask || !counts) return fail(STEM_E_INVALID_ARG, "scores, mask and counts must be non-NULL");
  if (score_row_stride < pl.max_n)
    return fail(STEM_E_INVALID_ARG, "score_row_stride = %lld < %d", (long long)score_row_stride, pl.max_n);
  if (mask_row_words < (pl.max_n + 31) / 32)
    return fail(STEM_E_INVALID_ARG, "mask_row_words = %d < %d", mask_row_words, (pl.max_n + 31) / 32);
  if (pl.max_n > 4096) return fail(STEM_E_UNSUPPORTED, "selection supports up to 4096 blocks per request");
  st = check_select_args(pl, rho_num, rho_den, mu_num, mu_den, mask, mask_row_words, counts);
  if (st != STEM_OK) return st;
  st = check_device();
  if (st != STEM_OK) return st;
  TopkArgs ta;
  ta.scores = scores;
  ta.stride = score_row_stride;
  ta.mask = mask;
  ta.mask_words = mask_row_words;
  ta.counts = counts;
  ta.NB = pl.NB;
  ta.hq = p->hq;
  ta.rho_num = rho_num;
  ta.rho_den = rho_den;
  ta.mu_num = mu_num;
  ta.mu_den = mu_den;
  ta.rt = pl.rt;
  return hip_status(launch_topk(ta, pl.max_n, p->num_reqs, (hipStream_t)stream), "topk launch");
}

// ---- the naive comparison path
static void naive_layout(const Plan& pl, int32_t samples, int64_t* row_stride, int64_t* mass_stride,
                         int64_t* rows_max, size_t* off_mass, size_t* total) {
  const stem_problem* p = pl.p;
  *row_stride = ((int64_t)pl.max_len + 63) / 64 * 64;
  *mass_stride = ((int64_t)pl.max_n + 63) / 64 * 64;
  *rows_max = (int64_t)pl.max_n * samples;
  const size_t buf = (size_t)p->hq * (size_t)(*rows_max) * (size_t)(*row_stride) * sizeof(float);
  const size_t mass = (size_t)p->hq * (size_t)(*rows_max) * (size_t)(*mass_stride) * sizeof(float);
  *off_mass = align256(buf);
  *total = *off_mass + align256(mass);
}

static int check_naive(const stem_problem* p, const Plan& pl, int32_t samples) {
  if (p->dtype != STEM_BF16 || p->kv_paged)
    return fail(STEM_E_UNSUPPORTED, "the naive comparison path supports bf16 inputs with contiguous K/V");
  if (samples < 1 || samples > p->block || p->block % samples != 0)
    return fail(STEM_E_INVALID_ARG, "samples = %d must divide block = %d", samples, p->block);
  (void)pl;
  return STEM_OK;
}

size_t stem_naive_workspace_bytes(const stem_problem* p, int32_t samples) {
  Plan pl;
  if (make_plan(p, &pl) != STEM_OK || check_naive(p, pl, samples) != STEM_OK) return 0;
  int64_t rs, ms, rm;
  size_t om, total;
  naive_layout(pl, samples, &rs, &ms, &rm, &om, &total);
  return total;
}

int stem_naive_score(const stem_problem* p, const void* q, const void* k, const void* v, float beta,
                     int32_t samples, float* scores, int64_t score_row_stride, void* ws, size_t ws_bytes,
                     void* naive_ws, size_t naive_ws_bytes, void* stream) {
  Plan pl;
  int st = make_plan(p, &pl);
  if (st != STEM_OK) return st;
  st = check_naive(p, pl, samples);
  if (st != STEM_OK) return st;
  if (!scores) return fail(STEM_E_INVALID_ARG, "scores must be non-NULL");
  if (score_row_stride < pl.max_n)
    return fail(STEM_E_INVALID_ARG, "score_row_stride = %lld < %d", (long long)score_row_stride, pl.max_n);
  st = check_pool_args(p, pl, q, k, v, beta, ws, ws_bytes);
  if (st != STEM_OK) return st;
  int64_t rs, ms, rm;
  size_t om_naive, need;
  naive_layout(pl, samples, &rs, &ms, &rm, &om_naive, &need);
  if (!naive_ws || naive_ws_bytes < need)
    return fail(STEM_E_WORKSPACE, "naive workspace of %zu bytes given, %zu needed",
                naive_ws ? naive_ws_bytes : (size_t)0, need);
  if (((uintptr_t)naive_ws & 255) != 0) return fail(STEM_E_WORKSPACE, "naive workspace must be 256-byte aligned");
  st = check_device();
  if (st != STEM_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_pooling(p, pl, q, k, v, ws, s);  // M (and the pooled q, k, unused here)
  if (e != hipSuccess) return hip_status(e, "pool launch");
  size_t oq, okk, om, wneed;
  layout(pl, &oq, &okk, &om, &wneed);
  NaiveArgs a;
  a.q = q;
  a.k = k;
  a.buf = (float*)naive_ws;
  a.mass = (float*)((char*)naive_ws + om_naive);
  a.M = (const float*)((char*)ws + om);
  a.scores = scores;
  a.row_stride = rs;
  a.mass_stride = ms;
  a.rows_max = rm;
  a.stride = score_row_stride;
  a.NB = pl.NB;
  a.hq = p->hq;
  a.hkv = p->hkv;
  a.d = p->head_dim;
  a.B = p->block;
  a.samples = samples;
  a.scale = 1.0f / sqrtf((float)p->head_dim);
  a.beta = beta;
  a.rt = pl.rt;
  int32_t lens[STEM_MAX_REQS], nbl[STEM_MAX_REQS];
  for (int r = 0; r < p->num_reqs; ++r) {
    lens[r] = p->cu_seqlens[r + 1] - p->cu_seqlens[r];
    nbl[r] = pl.rt.cu_blocks[r + 1] - pl.rt.cu_blocks[r];
  }
  return hip_status(launch_naive(a, lens, nbl, p->num_reqs, s), "naive launch");
}

static int prepare_bsa(const stem_problem* p, const void* q, const void* k, const void* v, const uint32_t* mask,
                       int32_t mask_row_words, float softmax_scale, void* out, float* lse, Plan* pl, BsaArgs* ba) {
  int st = make_plan(p, pl);
  if (st != STEM_OK) return st;
  if (!q || !k || !v || !out) return fail(STEM_E_INVALID_ARG, "q, k, v and out must be non-NULL");
  if (mask && mask_row_words < (pl->max_n + 31) / 32)
    return fail(STEM_E_INVALID_ARG, "mask_row_words = %d < %d", mask_row_words, (pl->max_n + 31) / 32);
  if (mask && pl->max_n > 2048) return fail(STEM_E_UNSUPPORTED, "masked attention supports up to 2048 blocks per request");
  if (!isfinite(softmax_scale)) return fail(STEM_E_INVALID_ARG, "softmax_scale is not finite");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15)
    return fail(STEM_E_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  ba->q = q;
  ba->k = k;
  ba->v = v;
  ba->mask = mask;
  ba->mask_words = mask ? mask_row_words : 0;
  ba->out = out;
  ba->lse = lse;
  ba->q_scale = p->q_scale;
  ba->k_scale = p->k_scale;
  ba->v_scale = p->v_scale;
  ba->hq = p->hq;
  ba->hkv = p->hkv;
  ba->B = p->block;
  ba->NB = pl->NB;
  ba->tokens = pl->tokens;
  const float sc = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)p->head_dim);
  ba->scale = sc;
  ba->scale_log2 = sc * 1.44269504088896340736f;
  ba->xcd_remap = ((int64_t)p->hq * pl->NB) % 8 == 0 ? 1 : 0;
  ba->kv = pl->kv;
  ba->rt = pl->rt;
  return STEM_OK;
}

int bsa_prefill(const stem_problem* p, const void* q, const void* k, const void* v, const uint32_t* mask,
                int32_t mask_row_words, float softmax_scale, void* out, float* lse, void* stream) {
  Plan pl;
  BsaArgs ba;
  int st = prepare_bsa(p, q, k, v, mask, mask_row_words, softmax_scale, out, lse, &pl, &ba);
  if (st != STEM_OK) return st;
  st = check_device();
  if (st != STEM_OK) return st;
  return hip_status(launch_bsa(ba, p->dtype, p->head_dim, p->kv_paged != 0, mask != nullptr, (hipStream_t)stream),
                    "bsa launch");
}

// V elements of the problem: every row of the contiguous tensor, or of the paged pool.
static int64_t v_elements(const stem_problem* p, const Plan& pl) {
  const int64_t rows = p->kv_paged ? (int64_t)p->num_pages * p->page_size : pl.tokens;
  return rows * p->hkv * p->head_dim;
}

size_t bsa_workspace_bytes(const stem_problem* p) {
  Plan pl;
  if (make_plan(p, &pl) != STEM_OK) return 0;
  ok();
  if (!bsa_fp8_supported(p->dtype, p->head_dim, p->block)) return 0;
  return (size_t)v_elements(p, pl) * 2;
}

int bsa_prefill_ws(const stem_problem* p, const void* q, const void* k, const void* v, const uint32_t* mask,
                   int32_t mask_row_words, float softmax_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                   void* stream) {
  Plan pl;
  BsaArgs ba;
  int st = prepare_bsa(p, q, k, v, mask, mask_row_words, softmax_scale, out, lse, &pl, &ba);
  if (st != STEM_OK) return st;
  const bool expand = bsa_fp8_supported(p->dtype, p->head_dim, p->block);
  const int64_t nv = expand ? v_elements(p, pl) : 0;
  if (expand) {
    if (!ws || ws_bytes < (size_t)nv * 2)
      return fail(STEM_E_WORKSPACE, "workspace of %zu bytes, bsa_workspace_bytes = %zu", ws ? ws_bytes : (size_t)0,
                  (size_t)nv * 2);
    if ((uintptr_t)ws & 15) return fail(STEM_E_INVALID_ARG, "ws must be 16-byte aligned");
  }
  st = check_device();
  if (st != STEM_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (!expand)
    return hip_status(launch_bsa(ba, p->dtype, p->head_dim, p->kv_paged != 0, mask != nullptr, s), "bsa launch");
  hipError_t e = launch_expand_fp8(v, ws, nv, s);
  if (e != hipSuccess) return hip_status(e, "V expansion launch");
  ba.v = ws;
  return hip_status(launch_bsa_fp8_vb16(ba, mask != nullptr, s), "bsa launch");
}

int bsa_prefill_inloop(const stem_problem* p, const void* q, const void* k, const void* v, const uint32_t* mask,
                       int32_t mask_row_words, float softmax_scale, void* out, float* lse, void* stream) {
  Plan pl;
  BsaArgs ba;
  if (!mask) return fail(STEM_E_INVALID_ARG, "the in-loop skip variant needs a mask");
  int st = prepare_bsa(p, q, k, v, mask, mask_row_words, softmax_scale, out, lse, &pl, &ba);
  if (st != STEM_OK) return st;
  if (!bsa_bf16_supported(p->dtype, p->head_dim, p->block) || p->kv_paged)
    return fail(STEM_E_UNSUPPORTED, "the in-loop skip variant supports bf16, head_dim 128, block 128, contiguous K/V");
  st = check_device();
  if (st != STEM_OK) return st;
  return hip_status(launch_bsa_bf16_inloop(ba, (hipStream_t)stream), "bsa in-loop launch");
}

}  // extern "C"
