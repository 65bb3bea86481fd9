// Fused OAM scoring and TPD top-k selection: the block scores of a row never leave the chip.
//
// Source: "从Stem稀疏注意力看大模型推理的架构取舍", section "HPC-Stem：评估选块，快几十倍" (scoring by one GEMM
// of compact block representations, and the budget and selection fused so that intermediate tensors do
// not go through HBM) and section "TPD：优先级排序" (the budget).
//
// One workgroup (4 wavefronts) owns kRows = 16 consecutive query-block rows i of one head h of one
// request.  Its 16 pooled query rows sit in LDS; each thread takes one column j and 8 of the rows at a
// time, streams kbar_j from memory (L2-resident: kbar of one KV head is n x d floats) and forms the dot
// products, writing the causal score rows S[i][j] = <qbar_i, kbar_j> / sqrt(d) + beta M[j] into LDS.  Then each wavefront
// selects 4 of the rows exactly as tpd_topk.hip does (same plan, same keys, same ties), reading the keys
// from LDS.  Each dot product is one fp32 FMA chain over d in increasing order
// followed by fmaf(acc, 1/sqrt(d), beta M[j]) -- the arithmetic of score_kernel -- so the scores, and
// therefore the masks, are bit-identical to the two-stage path.
// Bound: the fp32 FMAs of the causal dot products (4.3 GFLOP at 128K tokens and 32 heads) and the
// ballot rounds of the selection; HBM traffic is the pooled operands, the mask and the counts only.
#include "select_common.h"

namespace stem {

namespace {

constexpr int kRows = 16;
constexpr int kMaxD = 128;
constexpr int kWaves = 4;

template <int NS>
__global__ __launch_bounds__(kWaves * 64) void score_topk_kernel(ScoreTopkArgs a) {
  __shared__ float srow[kRows][64 * NS];
  __shared__ __align__(16) float qs[kRows][kMaxD];

  const int r = blockIdx.z;
  const int h = blockIdx.y;
  const int64_t cb = a.rt.cu_blocks[r];
  const int n = a.rt.cu_blocks[r + 1] - (int)cb;
  const int i0 = blockIdx.x * kRows;
  if (i0 >= n) return;  // uniform across the workgroup
  const int g = h / (a.hq / a.hkv);
  const int d = a.d;
  const int tid = threadIdx.x;
  const int ncols = min(i0 + kRows, n);  // causal bound of the workgroup's last row

  const float* qb = a.qbar + ((int64_t)h * a.NB + cb) * d;
  const float* kb = a.kbar + ((int64_t)g * a.NB + cb) * d;
  const float* Mg = a.M + (int64_t)g * a.NB + cb;

  // The workgroup's pooled query rows go to LDS once.  Each pass then covers 128 columns: wavefront w
  // takes columns c0 + 64 (w >> 1) + lane and the 8 rows 8 (w & 1) .. 8 (w & 1) + 7, forming their dot
  // products with kbar_j, d in increasing order; the query values are LDS broadcasts, kbar_j streams
  // through vector loads two steps ahead of its use.
  for (int e = tid; e < kRows * d; e += kWaves * 64) {
    const int row = e / d, col = e % d;
    qs[row][col] = qb[(int64_t)min(i0 + row, n - 1) * d + col];
  }
  __syncthreads();
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int rh = (wave & 1) * 8;
  const int nd4 = d / 4;  // 16 or 32
  for (int c0 = 0; c0 < ncols; c0 += 128) {
    const int j = c0 + (wave >> 1) * 64 + lane;
    const int jj = min(j, ncols - 1);  // lanes past the last column recompute it (not stored)
    float acc[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] = 0.f;
    const float4* kr = (const float4*)(kb + (int64_t)jj * d);
    float4 kv0 = kr[0], kv1 = kr[1];
    for (int d4 = 0; d4 < nd4; d4 += 2) {
      const float4 ka = kv0, kc = kv1;
      if (d4 + 2 < nd4) {
        kv0 = kr[d4 + 2];
        kv1 = kr[d4 + 3];
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const float4 qv = *(const float4*)&qs[rh + x][4 * d4];
        acc[x] = fmaf(qv.x, ka.x, acc[x]);
        acc[x] = fmaf(qv.y, ka.y, acc[x]);
        acc[x] = fmaf(qv.z, ka.z, acc[x]);
        acc[x] = fmaf(qv.w, ka.w, acc[x]);
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const float4 qv = *(const float4*)&qs[rh + x][4 * d4 + 4];
        acc[x] = fmaf(qv.x, kc.x, acc[x]);
        acc[x] = fmaf(qv.y, kc.y, acc[x]);
        acc[x] = fmaf(qv.z, kc.z, acc[x]);
        acc[x] = fmaf(qv.w, kc.w, acc[x]);
      }
    }
    const float bm = a.beta * Mg[jj];
#pragma unroll
    for (int x = 0; x < 8; ++x)
      if (j < ncols && j <= i0 + rh + x) srow[rh + x][j] = fmaf(acc[x], a.inv_sqrt_d, bm);
  }
  __syncthreads();

  // ---- selection: wavefront w takes rows 4w .. 4w + 3 of the workgroup
  const TpdPlan plan = wave_plan(n, a.rho_num, a.rho_den, a.mu_num, a.mu_den, lane);
  for (int rr = 0; rr < kRows / kWaves; ++rr) {
    const int lr = wave * (kRows / kWaves) + rr;
    const int i = i0 + lr;
    if (i >= n) break;
    const int64_t row = (int64_t)h * a.NB + cb + i;
    const int k = (int)tpd_row_budget(plan, i);
    const int nslot = i / 64 + 1;
    uint32_t key[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j = lane + 64 * s;
      key[s] = (s < nslot && j <= i) ? ord_key(srow[lr][j]) : 0u;
    }
    select_row<NS>(key, nslot, k, lane, a.mask + row * a.mask_words, a.mask_words);
    if (lane == 0) a.counts[row] = k;
  }
}

}  // namespace

hipError_t launch_score_topk(const ScoreTopkArgs& a, int max_n, int num_reqs, hipStream_t s) {
  dim3 grid((unsigned)((max_n + kRows - 1) / kRows), (unsigned)a.hq, (unsigned)num_reqs);
  dim3 block(kWaves * 64);
  if (max_n <= 64) hipLaunchKernelGGL(score_topk_kernel<1>, grid, block, 0, s, a);
  else if (max_n <= 128) hipLaunchKernelGGL(score_topk_kernel<2>, grid, block, 0, s, a);
  else if (max_n <= 256) hipLaunchKernelGGL(score_topk_kernel<4>, grid, block, 0, s, a);
  else if (max_n <= 512) hipLaunchKernelGGL(score_topk_kernel<8>, grid, block, 0, s, a);
  else if (max_n <= 1024) hipLaunchKernelGGL(score_topk_kernel<16>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(score_topk_kernel<32>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace stem
