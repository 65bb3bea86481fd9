/*
 * stem.h -- C ABI of the Stem sparse-attention prefill path on AMD Instinct MI355X (gfx950).
 *
 * The path has three stages, all run by HIP kernels enqueued on the caller's stream:
 *   stem_score     Output-Aware Metric (OAM) block scores from compact per-block Q/K representations and
 *                  one GEMM, plus beta * log||V_j||_2.
 *                  Source: "从Stem稀疏注意力看大模型推理的架构取舍" (developer.cloud.tencent.cn/article/
 *                  2709440), sections "OAM：价值评估" and "HPC-Stem：评估选块，快几十倍".
 *   stem_tpd_topk  Token Position Decay (TPD) budgets fused with per-row top-k block selection.
 *                  Source: same page, sections "TPD：优先级排序" and "HPC-Stem：评估选块，快几十倍".
 *   bsa_prefill    Block-sparse causal flash attention over a compacted per-row list of selected KV
 *                  blocks (skipped blocks behave as -inf scores); or dense causal attention when no mask
 *                  is given.  Source: same page, section "HPC-BSA：跳块零开销的秘密" (including its
 *                  paged-KV-cache paragraph).
 * Variants of the same stages, declared below with their own notes:
 *   stem_score_select     stem_score and stem_tpd_topk in one pass, without the score tensor.
 *   stem_quantize_score   W8A8: bf16 Q/K/V to per-head-scaled e4m3 codes, pooled in the same pass, scored.
 *   stem_quantize_fp8     the quantisation alone (the unfused baseline of stem_quantize_score).
 *   stem_score_noalloc    stem_score with its pooled tensors in a static per-device scratch.
 *   bsa_prefill_ws        bsa_prefill with a workspace (fp8: V expanded to bf16 once per call).
 *   bsa_prefill_inloop    bsa_prefill with the skip test inside the loop (a comparison path).
 *   stem_naive_score      token-level softmax scoring of sampled queries (a comparison path).
 *
 * Conventions (all entry points):
 *   - Plain C types only.  `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Device pointers are marked DEVICE, host pointers HOST.  The caller owns every buffer; the library
 *     never allocates or frees memory and never synchronises.  Launches are asynchronous: results are
 *     ready when the stream reaches them.
 *   - Every argument is validated on the host before anything is enqueued.  On failure the function
 *     returns a negative STEM_E_* status, enqueues nothing, and stem_last_error() (per thread) describes
 *     the problem.  STEM_E_HIP means a HIP runtime call failed (message included).
 *   - Only gfx950 devices are accepted (STEM_E_UNSUPPORTED otherwise).
 *
 * Tensor layouts (row-major, innermost last):
 *   Q         [tokens][hq][head_dim]        tokens = cu_seqlens[num_reqs] (requests packed back to back)
 *   K, V      contiguous: [tokens][hkv][head_dim]
 *             paged:      [num_pages][page_size][hkv][head_dim]; request r's token t is in physical page
 *                         page_table[r * page_table_stride + t / page_size], slot t % page_size
 *   element   STEM_F32 float; STEM_BF16 bfloat16 bits; STEM_FP8_E4M3 OCP e4m3fn codes whose real value is
 *             code * scale[head] (q_scale per query head, k_scale / v_scale per KV head, float)
 *   O         [tokens][hq][head_dim], float for STEM_F32, bfloat16 otherwise
 *   LSE       [hq][tokens] float, natural-log log-sum-exp of the scaled logits of each query row
 *   blocks    request r has n_r = ceil(len_r / block) query blocks = KV blocks; blocks of all requests
 *             are numbered globally, request by request (NB = sum n_r); j is the block index inside its
 *             request
 *   scores    float, row (h, global block ib) at scores + (h * NB + ib) * score_row_stride; entry j holds
 *             S[h][i][j] for j <= i (i = ib's index inside its request); entries j > i are not written
 *   mask      uint32, row (h, ib) at mask + (h * NB + ib) * mask_row_words; bit j (word j/32, bit j%32)
 *             set = KV block j selected; bits j > i are ignored by bsa_prefill and written 0 by
 *             stem_tpd_topk
 *   counts    int32 [hq][NB]: number of blocks selected in each row (the TPD budget k_i of the row)
 *   GQA       query head h reads KV head h / (hq / hkv)
 */
#ifndef STEM_H
#define STEM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum stem_status {
  STEM_OK = 0,
  STEM_E_INVALID_ARG = -1, /* a pointer, size, shape or parameter is invalid */
  STEM_E_UNSUPPORTED = -2, /* valid but not supported here (dtype/shape combination, non-gfx950 device) */
  STEM_E_WORKSPACE = -3,   /* workspace missing or smaller than stem_workspace_bytes() */
  STEM_E_HIP = -4          /* a HIP runtime call failed */
};

enum stem_dtype { STEM_F32 = 0, STEM_BF16 = 1, STEM_FP8_E4M3 = 2 };

#define STEM_MAX_REQS 256 /* requests per call */
#define STEM_SCRATCH_BYTES (64u << 20) /* static scratch of stem_score_noalloc, per device */

/* Problem descriptor shared by all entry points.  Read during the call only. */
typedef struct stem_problem {
  int32_t num_reqs;          /* 1..STEM_MAX_REQS */
  const int32_t* cu_seqlens; /* HOST [num_reqs + 1]: 0 = cu[0] <= cu[1] <= ...; len_r = cu[r+1] - cu[r] */
  int32_t hq, hkv;           /* query / KV heads, hq % hkv == 0 */
  int32_t head_dim;          /* 64 or 128 */
  int32_t block;             /* block size B in tokens: 64 or 128 */
  int32_t dtype;             /* enum stem_dtype of Q, K and V */
  int32_t kv_paged;          /* 0: contiguous K/V; 1: paged K/V */
  int32_t page_size;         /* paged only: tokens per page, a multiple of 16 */
  int32_t num_pages;         /* paged only: pages in the K and V pools */
  const int32_t* page_table; /* paged only, DEVICE [num_reqs][page_table_stride]: physical page ids */
  int32_t page_table_stride; /* paged only: >= ceil(max len_r / page_size) */
  const float* q_scale;      /* fp8 only, DEVICE [hq] */
  const float* k_scale;      /* fp8 only, DEVICE [hkv] */
  const float* v_scale;      /* fp8 only, DEVICE [hkv] */
} stem_problem;

/* Pure host helpers --------------------------------------------------------------------------------- */

/* Validates `p` and reports NB (total blocks) and the largest per-request block count. */
int stem_block_counts(const stem_problem* p, int64_t* total_blocks, int32_t* max_blocks);

/* Workspace bytes that stem_score needs (0 on invalid input; see stem_last_error()).  The workspace holds,
 * at the offsets returned by stem_workspace_layout, q-bar float [hq][NB][head_dim], k-bar float
 * [hkv][NB][head_dim] and M float [hkv][NB] (the block means of Q, K and ln||v||). */
size_t stem_workspace_bytes(const stem_problem* p);
int stem_workspace_layout(const stem_problem* p, size_t* off_qbar, size_t* off_kbar, size_t* off_m);

/* TPD budgets of one request with n blocks, written to HOST k_out[n] (same arithmetic as the kernel).
 * Budget fraction rho = rho_num/rho_den in [0, 1]; decay ratio mu = mu_num/mu_den in (0, 1].
 * Total T = round-half-up(rho * n(n+1)/2) clamped to [n, n(n+1)/2].  Row i (0-based) has the linear
 * weight w_i = 1 - (1 - mu) i/(n-1); its real budget is r_i = min(max(x w_i, 1), i+1) with x solving
 * sum r_i = T; integer budgets round the prefix sums: k_i = floor(P_i + 1/2) - floor(P_{i-1} + 1/2).
 * Source: "TPD：优先级排序" (linear decay from k_start to k_end = mu k_start, total unchanged). */
int stem_tpd_budgets_host(int32_t n, int32_t rho_num, int32_t rho_den, int32_t mu_num, int32_t mu_den,
                          int32_t* k_out);

const char* stem_status_string(int status);
const char* stem_last_error(void); /* message of this thread's last failed call ("" if none) */

/* Stage 1: OAM block scores ----------------------------------------------------------------------- */
/* S[h][i][j] = <qbar_{h,i}, kbar_{g,j}> / sqrt(head_dim) + beta * M[g][j] for j <= i, g = h/(hq/hkv),
 * where qbar/kbar are the means of Q/K over the valid tokens of a block and M[g][j] is the mean over
 * block j's tokens of ln||v_t||_2 (natural log).  q, k, v: DEVICE (layouts above).  scores: DEVICE,
 * score_row_stride >= max n_r.  ws: DEVICE workspace of ws_bytes >= stem_workspace_bytes(p), 256-byte
 * aligned; the pooled tensors stay there after the call. */
int stem_score(const stem_problem* p, const void* q, const void* k, const void* v, float beta, float* scores,
               int64_t score_row_stride, void* ws, size_t ws_bytes, void* stream);

/* Stage 2: fused TPD budget + top-k selection ------------------------------------------------------ */
/* For each row (h, ib): k_i from the TPD budget of ib's request (see stem_tpd_budgets_host), then the k_i
 * largest scores among j <= i; equal scores go to the lower j.  Writes the packed mask row (all
 * mask_row_words words, zero past i) and counts[h * NB + ib] = k_i.  scores: DEVICE as written by
 * stem_score; mask: DEVICE, mask_row_words >= ceil(max n_r / 32); counts: DEVICE int32 [hq][NB]. */
int stem_tpd_topk(const stem_problem* p, const float* scores, int64_t score_row_stride, int32_t rho_num,
                  int32_t rho_den, int32_t mu_num, int32_t mu_den, uint32_t* mask, int32_t mask_row_words,
                  int32_t* counts, void* stream);

/* Stage 1 without a workspace, for callers that cannot allocate device memory (code being captured
 * into a HIP graph, tight serving loops, harnesses that forbid allocation).  Same arguments, kernels and
 * results as stem_score, minus ws/ws_bytes: the pooled q-bar, k-bar and M go to a static scratch array
 * the library holds in each device's memory (STEM_SCRATCH_BYTES, allocated when the library's code is
 * loaded on the device and kept until the process ends; nothing is allocated by the call).  A problem
 * whose workspace (stem_workspace_bytes) exceeds STEM_SCRATCH_BYTES is rejected with STEM_E_UNSUPPORTED
 * before anything is enqueued; 64 MiB holds up to 3,271 blocks (418K tokens at block 128) of a layer with
 * 32 query / 8 KV heads of head_dim 128.
 * Every call on a device shares that device's scratch and leaves its pooled tensors there: calls that
 * may overlap on one device (several streams or threads) race, so serialise them. */
int stem_score_noalloc(const stem_problem* p, const void* q, const void* k, const void* v, float beta,
                       float* scores, int64_t score_row_stride, void* stream);

/* Stage 1 for an fp8 (W8A8) layer from bf16 activations: quantisation fused with pooling -------------- */
/* q, k, v: DEVICE bf16 in the layouts above (contiguous K/V).  Writes the per-head scales
 * q_scale[hq], k_scale[hkv], v_scale[hkv] (DEVICE; scale = amax / 448 in fp32, 1 for an all-zero head),
 * the e4m3fn codes q8, k8, v8 (DEVICE, same layouts; code = round-to-nearest-even of x / scale clamped to
 * +-448), and then exactly what stem_score computes from those codes and scales (pooled workspace and
 * block scores), without reading the codes back: the pooling works on the values it has just quantised.
 * p describes the fp8 layer (dtype STEM_FP8_E4M3, contiguous K/V); its own scale pointers are not read
 * here (they are normally these same output arrays, for the later stages).
 * Source: "答案不在算法里" (W8A8-FP8 deployment) with "HPC-Stem：评估选块，快几十倍" (fusing to avoid passes
 * through HBM). */
int stem_quantize_score(const stem_problem* p, const void* q, const void* k, const void* v, void* q8, void* k8,
                        void* v8, float* q_scale, float* k_scale, float* v_scale, float beta, float* scores,
                        int64_t score_row_stride, void* ws, size_t ws_bytes, void* stream);

/* W8A8 quantisation alone: the first half of stem_quantize_score without the pooling.  Same inputs,
 * scales and codes (bit for bit); reads the bf16 inputs twice (per-head amax, then the codes) and writes
 * the codes once.  stem_score on its outputs then gives what stem_quantize_score gives.  It exists as the
 * unfused baseline of that fusion, and for callers that quantise without scoring.
 * Source: "答案不在算法里" (W8A8-FP8 deployment). */
int stem_quantize_fp8(const stem_problem* p, const void* q, const void* k, const void* v, void* q8, void* k8,
                      void* v8, float* q_scale, float* k_scale, float* v_scale, void* stream);

/* Stages 1 + 2 fused: the score tensor never reaches memory ---------------------------------------- */
/* Pools Q/K/V into the workspace exactly as stem_score does, then computes each row's block scores on
 * chip and selects from them exactly as stem_tpd_topk does: mask and counts are bit-identical to
 * stem_score followed by stem_tpd_topk with the same arguments, without the score tensor (NB x max n
 * floats per query head) being written or read.  Arguments as in those two calls; requests of up to 2048
 * blocks (STEM_E_UNSUPPORTED beyond).
 * Source: "HPC-Stem：评估选块，快几十倍" (scoring, budget and selection fused so that no intermediate tensor
 * goes through HBM). */
int stem_score_select(const stem_problem* p, const void* q, const void* k, const void* v, float beta,
                      int32_t rho_num, int32_t rho_den, int32_t mu_num, int32_t mu_den, uint32_t* mask,
                      int32_t mask_row_words, int32_t* counts, void* ws, size_t ws_bytes, void* stream);

/* Comparison path: the naive, token-level form of the block score ----------------------------------- */
/* For `samples` sampled queries per block (block i's sample s is token min(i*block + s*block/samples,
 * L - 1)), the softmax of q_t . k_tau / sqrt(head_dim) over the keys tau <= t, the probability mass per key
 * block j, averaged over block i's samples: S[h][i][j] = ln(mean mass) + beta * M[g][j] for j <= i, in
 * stem_score's layout (stem_tpd_topk selects from it as usual).  Every step goes through memory: the
 * token-level logits and probabilities (hq x max_n*samples x max L floats) live in naive_ws, DEVICE,
 * naive_ws_bytes >= stem_naive_workspace_bytes(p, samples), 256-byte aligned; ws is stem_score's
 * workspace (M is pooled there).  bf16 inputs with contiguous K/V only; samples must divide block.
 * It exists to measure what the pooled one-GEMM scoring saves.
 * Source: "HPC-Stem：评估选块，快几十倍" (the direct token-level computation needs intermediate tensors of
 * tens of GB and is tens of times slower). */
size_t stem_naive_workspace_bytes(const stem_problem* p, int32_t samples); /* 0 on invalid input */
int stem_naive_score(const stem_problem* p, const void* q, const void* k, const void* v, float beta,
                     int32_t samples, float* scores, int64_t score_row_stride, void* ws, size_t ws_bytes,
                     void* naive_ws, size_t naive_ws_bytes, void* stream);

/* Stage 3: block-sparse attention ----------------------------------------------------------------- */
/* For query token t of query block i, head h: out = softmax over visible keys s of (q_t . k_s) * scale,
 * applied to v_s, where s is visible when its block j is selected in mask row (h, i) (j <= i) and s <= t
 * inside the same request.  mask == NULL runs dense causal attention (every j <= i visible).  Rows with
 * no visible key get out = 0 and lse = -inf.  softmax_scale <= 0 means 1/sqrt(head_dim).  q, k, v, out:
 * DEVICE (layouts above); lse: DEVICE or NULL.  fp8 logits use q_scale[h] * k_scale[g] and outputs
 * v_scale[g]. */
int bsa_prefill(const stem_problem* p, const void* q, const void* k, const void* v, const uint32_t* mask,
                int32_t mask_row_words, float softmax_scale, void* out, float* lse, void* stream);

/* Workspace bytes that bsa_prefill_ws needs: 2 bytes per V element (V's bf16 expansion) for fp8 problems
 * of head_dim 128 and block 128 -- contiguous: tokens * hkv * head_dim elements; paged: num_pages *
 * page_size * hkv * head_dim -- and 0 for every other problem (0 also on invalid input; see
 * stem_last_error()). */
size_t bsa_workspace_bytes(const stem_problem* p);

/* bsa_prefill with a caller workspace; same arguments, outputs and limits otherwise.  For fp8 problems of
 * head_dim 128 and block 128 it first expands V's e4m3 codes to bfloat16 into ws (exact: every e4m3 value
 * is a bfloat16 value; v_scale still applies at the output), then runs the attention on that copy, which
 * reaches LDS by direct loads instead of a conversion on every visit of a V tile; the outputs are bit for
 * bit those of bsa_prefill.  Every other problem ignores ws and runs exactly as bsa_prefill.  ws: DEVICE,
 * 16-byte aligned, ws_bytes >= bsa_workspace_bytes(p) (STEM_E_WORKSPACE otherwise), not overlapping the
 * other buffers; it holds the bf16 V after the call.
 * Source: "HPC-BSA：跳块零开销的秘密" (FP8 compute throughput) and "答案不在算法里" (W8A8-FP8). */
int bsa_prefill_ws(const stem_problem* p, const void* q, const void* k, const void* v, const uint32_t* mask,
                   int32_t mask_row_words, float softmax_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                   void* stream);

/* Comparison variant of bsa_prefill with the skip decision inside the loop: instead of building each
 * row's list of selected blocks, it walks every causal block j <= i and tests j's mask bit at each step,
 * skipping the loads and the compute of unselected blocks but not the step.  Same arguments and same
 * outputs as bsa_prefill (bit for bit: the selected blocks see the same arithmetic in the same order);
 * it exists to measure what building the list saves.  mask must be non-NULL; only bf16, head_dim 128,
 * block 128 and contiguous K/V are supported (STEM_E_UNSUPPORTED otherwise).
 * Source: "HPC-BSA：跳块零开销的秘密" (a skip test inside the inner loop costs divergence and pipeline
 * bubbles; the list moves the decision out of the loop). */
int bsa_prefill_inloop(const stem_problem* p, const void* q, const void* k, const void* v, const uint32_t* mask,
                       int32_t mask_row_words, float softmax_scale, void* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* STEM_H */
