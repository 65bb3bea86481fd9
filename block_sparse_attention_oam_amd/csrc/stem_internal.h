// Internal launch interface between the C-ABI host code and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "stem_common.h"
#include "tpd_budget.h"

namespace stem {

// Everything a launcher needs, validated and derived on the host.
struct Plan {
  const stem_problem* p;
  ReqTable rt;
  int64_t NB;        // total blocks
  int32_t max_n;     // largest per-request block count
  int32_t max_len;   // longest request
  int64_t tokens;
  KvAddr kv;
};

struct PoolArgs {
  const void* q;  // inputs (bf16 sources when quantising)
  const void* k;
  const void* v;
  void* q8;       // quantising pool only: e4m3fn outputs in the same layouts
  void* k8;
  void* v8;
  float* qbar;
  float* kbar;
  float* M;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  int32_t hq, hkv, d, B;
  int64_t NB;
  int32_t q_chunks, kv_chunks;
  KvAddr kv;
  ReqTable rt;
};

struct ScoreArgs {
  const float* qbar;
  const float* kbar;
  const float* M;
  float* scores;
  int64_t stride;
  int64_t NB;
  int32_t hq, hkv, d;
  float beta, inv_sqrt_d;
  ReqTable rt;
};

struct TopkArgs {
  const float* scores;
  int64_t stride;
  uint32_t* mask;
  int32_t mask_words;
  int32_t* counts;
  int64_t NB;
  int32_t hq;
  int32_t rho_num, rho_den, mu_num, mu_den;
  ReqTable rt;
};

struct ScoreTopkArgs {
  const float* qbar;
  const float* kbar;
  const float* M;
  uint32_t* mask;
  int32_t mask_words;
  int32_t* counts;
  int64_t NB;
  int32_t hq, hkv, d;
  float beta, inv_sqrt_d;
  int32_t rho_num, rho_den, mu_num, mu_den;
  ReqTable rt;
};

struct NaiveArgs {
  const void* q;
  const void* k;
  float* buf;     // [hq][rows_max][row_stride] logits, then probabilities
  float* mass;    // [hq][rows_max][mass_stride] per-block probability mass
  const float* M; // pooled ln||v|| means [hkv][NB]
  float* scores;  // [hq][NB][stride]
  int64_t row_stride, mass_stride, rows_max, stride, NB;
  int32_t hq, hkv, d, B, samples;
  float scale, beta;
  ReqTable rt;
};

struct BsaArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint32_t* mask;
  int32_t mask_words;
  void* out;
  float* lse;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  int32_t hq, hkv, B;
  int64_t NB;
  int64_t tokens;
  float scale_log2;  // softmax scale * log2(e)
  float scale;       // softmax scale
  int32_t xcd_remap; // 1: blockIdx -> (kv head, block, head) remap is active
  KvAddr kv;
  ReqTable rt;
};

hipError_t launch_pool(const PoolArgs& a, int dtype, hipStream_t s);
// bf16 inputs -> per-head amax into the scale arrays, scales, then the quantising pool (fp8 codes out).
hipError_t launch_quant_pool(const PoolArgs& a, float* q_scale, float* k_scale, float* v_scale, int64_t tokens,
                             hipStream_t s);
// bf16 inputs -> per-head scales and e4m3fn codes, no pooling.
hipError_t launch_quant(const PoolArgs& a, float* q_scale, float* k_scale, float* v_scale, int64_t tokens,
                        hipStream_t s);
hipError_t launch_score(const ScoreArgs& a, int max_n, int num_reqs, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, int max_n, int num_reqs, hipStream_t s);
hipError_t launch_score_topk(const ScoreTopkArgs& a, int max_n, int num_reqs, hipStream_t s);
hipError_t launch_naive(const NaiveArgs& a, const int32_t* lens, const int32_t* nblocks, int num_reqs,
                        hipStream_t s);
hipError_t launch_bsa(const BsaArgs& a, int dtype, int head_dim, bool paged, bool masked, hipStream_t s);
bool bsa_bf16_supported(int dtype, int head_dim, int block);
hipError_t launch_bsa_bf16(const BsaArgs& a, bool masked, hipStream_t s);
hipError_t launch_bsa_bf16_inloop(const BsaArgs& a, hipStream_t s);
bool bsa_fp8_supported(int dtype, int head_dim, int block);
hipError_t launch_bsa_fp8(const BsaArgs& a, bool masked, hipStream_t s);
// fp8 attention reading V expanded to bf16 (a.v), and the expansion itself (n codes, a multiple of 16).
hipError_t launch_bsa_fp8_vb16(const BsaArgs& a, bool masked, hipStream_t s);
hipError_t launch_expand_fp8(const void* v_codes, void* v_bf16, int64_t n, hipStream_t s);

}  // namespace stem
