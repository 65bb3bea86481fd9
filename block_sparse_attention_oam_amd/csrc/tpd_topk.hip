// Stage 2 kernel: Token Position Decay budget fused with top-k block selection.
//
// Source: "从Stem稀疏注意力看大模型推理的架构取舍", sections "TPD：优先级排序" (linear decay of the per-position
// top-k budget from k_start to k_end = mu k_start, same total as a uniform budget) and "HPC-Stem：评估选块，
// 快几十倍" (budget generation is one formula per position and is fused with the selection sort, so no
// budget tensor goes through HBM).
//
// One wavefront handles 2-8 query-block rows (h, i) of one request (chosen at launch), i = i0, i0 + stride, ...
// (strided, so that every wave gets a similar mix of short and long rows; the next row's scores are
// loaded while the current row is selected):
//   1. the request's budget plan (capped prefix / linear middle / floored suffix, tpd_budget.h) is solved
//      by a 64-way parallel search: each lane evaluates one breakpoint predicate, a ballot picks the
//      sub-interval, about log_64(n) rounds;
//   2. per row, k_i comes from the closed form of the rounded prefix sums;
//   3. the row's scores (j <= i, lane l holds j = l + 64 s) become order-preserving uint32 keys and the
//      k-th largest key is found bit by bit (MSB first) with ballot + popcount counts;
//   4. keys above the threshold are selected, then equal keys in increasing j until k are taken (ties go
//      to the lower block index); each ballot is directly two 32-bit words of the packed mask row.
// Bound: reading the causal half of the score rows (HBM) plus ~32 ballot rounds per row (ALU).
#include "select_common.h"

namespace stem {

namespace {

constexpr int kWaves = 4;
// Rows per wave: enough waves to cover the chip's latency (about 4096 in all), at most 8 rows each.  On
// the 32K layer (8192 rows) 2 rows per wave run the kernel 1.6x faster than 8; from 128K on, 8 is as fast
// as fewer or faster.
constexpr int kMaxRowsPerWave = 8;
constexpr int kMinRowsPerWave = 2;
constexpr int64_t kTargetWaves = 4096;

template <int NS>
__global__ __launch_bounds__(kWaves * 64) void topk_kernel(TopkArgs a) {
  const int r = blockIdx.z;
  const int h = blockIdx.y;
  const int64_t cb = a.rt.cu_blocks[r];
  const int n = a.rt.cu_blocks[r + 1] - (int)cb;
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  // rows i_begin, i_begin + stride, ... (a mix of short and long rows per wave)
  const int i_begin = blockIdx.x * kWaves + wave;
  const int stride = gridDim.x * kWaves;
  if (i_begin >= n) return;
  const TpdPlan plan = wave_plan(n, a.rho_num, a.rho_den, a.mu_num, a.mu_den, lane);

  // raw scores of the next row are loaded while the current row is selected
  float nxt[NS];
  auto load_row = [&](int i, float* v) {
    const float* srow = a.scores + ((int64_t)h * a.NB + cb + i) * a.stride;
    const int nslot = i / 64 + 1;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j = lane + 64 * s;
      v[s] = (s < nslot && j <= i) ? srow[j] : 0.f;
    }
  };
  load_row(i_begin, nxt);
  for (int i = i_begin; i < n; i += stride) {
    const int64_t row = (int64_t)h * a.NB + cb + i;
    const int nslot = i / 64 + 1;
    uint32_t key[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j = lane + 64 * s;
      key[s] = (s < nslot && j <= i) ? ord_key(nxt[s]) : 0u;
    }
    if (i + stride < n) load_row(i + stride, nxt);
    const int k = (int)tpd_row_budget(plan, i);
    select_row<NS>(key, nslot, k, lane, a.mask + row * a.mask_words, a.mask_words);
    if (lane == 0) a.counts[row] = k;
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, int max_n, int num_reqs, hipStream_t s) {
  const int64_t rows = (int64_t)a.hq * max_n * num_reqs;
  const int rpw = (int)std::min<int64_t>(kMaxRowsPerWave, std::max<int64_t>(kMinRowsPerWave, rows / kTargetWaves));
  const int rows_per_wg = kWaves * rpw;
  dim3 grid((unsigned)((max_n + rows_per_wg - 1) / rows_per_wg), (unsigned)a.hq, (unsigned)num_reqs);
  dim3 block(kWaves * 64);
  if (max_n <= 64) hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, s, a);
  else if (max_n <= 128) hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, s, a);
  else if (max_n <= 256) hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, a);
  else if (max_n <= 512) hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, a);
  else if (max_n <= 1024) hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, a);
  else if (max_n <= 2048) hipLaunchKernelGGL(topk_kernel<32>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(topk_kernel<64>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace stem
