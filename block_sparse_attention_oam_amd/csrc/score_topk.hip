// Fused OAM scoring and TPD top-k selection: the block scores of a row never leave the chip.
//
// Source: "从Stem稀疏注意力看大模型推理的架构取舍", section "HPC-Stem：评估选块，快几十倍" (scoring by one GEMM
// of compact block representations, and the budget and selection fused so that intermediate tensors do
// not go through HBM) and section "TPD：优先级排序" (the budget).
//
// One workgroup owns kRows = 16 consecutive query-block rows i of one request for two query heads of the
// same KV group (one head when the group size is odd), 4 wavefronts per head; wavefront w of a head computes
// and then selects rows 4w .. 4w + 3.  Lane l holds columns j = l + 64 s of those rows in registers, so the
// score rows never leave the wavefront: each dot product is one fp32 FMA chain over d in increasing order
// followed by fmaf(acc, 1/sqrt(d), beta M[j]) -- the arithmetic of score_kernel -- so the scores, and
// therefore the masks, are bit-identical to the two-stage path.  The key representations kbar_j
// (L2-resident: n x d floats per KV head) pass through LDS once per workgroup, 16 dimensions at a time
// (float4-major, so the lanes' 16-byte reads are conflict-free), and serve both heads; the pooled query
// rows are LDS broadcasts, read four dimensions at a time (which keeps the kernel at 4 wavefronts per SIMD
// for n <= 1024 blocks).  Selection then runs on the registers exactly as tpd_topk.hip does (same plan,
// same keys, same ties).  Workgroups of the longest rows are dispatched first.
// Bound: the fp32 FMAs of the causal dot products (4.3 GFLOP at 128K tokens and 32 heads) and the
// ballot rounds of the selection; HBM traffic is the pooled operands, the mask and the counts only.
#include "select_common.h"

namespace stem {

namespace {

constexpr int kRows = 16;
constexpr int kMaxD = 128;
constexpr int kWavesPerHead = 4;
constexpr int kRowsPerWave = kRows / kWavesPerHead;

// HEADS query heads of one KV group share the workgroup (and its staged kbar): 4 HEADS wavefronts.
template <int NS, int HEADS>
__global__ __launch_bounds__(HEADS * kWavesPerHead * 64) void score_topk_kernel(ScoreTopkArgs a) {
  constexpr int kThreads = HEADS * kWavesPerHead * 64;
  // dimensions of kbar staged per pass: 16 when two heads share the staging and n <= 1024 blocks (80 KB of
  // LDS, two workgroups per CU), else 8
  constexpr int kDc = (HEADS == 2 && NS <= 16) ? 16 : 8;
  __shared__ float4 ks[kDc / 4][64 * NS];  // ks[hh][j] = kbar_j[d0 + 4 hh .. d0 + 4 hh + 3]
  __shared__ __align__(16) float qs[HEADS][kRows][kMaxD];

  const int r = blockIdx.z;
  const int hfirst = blockIdx.x * HEADS;  // heads vary fastest in dispatch order, row blocks from the last one back
  const int64_t cb = a.rt.cu_blocks[r];
  const int n = a.rt.cu_blocks[r + 1] - (int)cb;
  const int nblk = (n + kRows - 1) / kRows;
  const int rb = nblk - 1 - (int)blockIdx.y;
  if (rb < 0) return;  // uniform across the workgroup (a shorter request of the batch)
  const int i0 = rb * kRows;
  const int g = hfirst / (a.hq / a.hkv);
  const int d = a.d;
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int hw = wave / kWavesPerHead;  // this wave's head within the workgroup
  const int wr = wave % kWavesPerHead;  // and its quarter of the rows
  const int h = hfirst + hw;
  const int ncols = min(i0 + kRows, n);                 // causal bound of the workgroup's last row
  const int wfirst = i0 + kRowsPerWave * wr;            // this wave's first row
  const int wlast = min(wfirst + kRowsPerWave, n) - 1;  // and its last
  const int wslot = wfirst >= n ? 0 : wlast / 64 + 1;   // column slots this wave needs

  const float* kb = a.kbar + ((int64_t)g * a.NB + cb) * d;
  const float* Mg = a.M + (int64_t)g * a.NB + cb;

  for (int e = tid; e < HEADS * kRows * d; e += kThreads) {
    const int hh = e / (kRows * d), row = (e / d) % kRows, col = e % d;
    const float* qb = a.qbar + ((int64_t)(hfirst + hh) * a.NB + cb) * d;
    qs[hh][row][col] = qb[(int64_t)min(i0 + row, n - 1) * d + col];
  }

  float acc[kRowsPerWave][NS];
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr)
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[rr][s] = 0.f;
  const int rbase = wr * kRowsPerWave;
  for (int d0 = 0; d0 < d; d0 += kDc) {
    __syncthreads();  // the previous chunk's reads are done (and, on the first pass, qs is written)
    for (int e = tid; e < ncols * (kDc / 4); e += kThreads) {
      const int j = e / (kDc / 4), hh = e % (kDc / 4);
      ks[hh][j] = *(const float4*)(kb + (int64_t)j * d + d0 + 4 * hh);
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < kDc / 4; ++hh) {  // four dimensions at a time: fewer live registers
      float q[kRowsPerWave][4];
#pragma unroll
      for (int rr = 0; rr < kRowsPerWave; ++rr) {
        const float4 v = *(const float4*)&qs[hw][rbase + rr][d0 + 4 * hh];
        q[rr][0] = v.x;
        q[rr][1] = v.y;
        q[rr][2] = v.z;
        q[rr][3] = v.w;
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s < wslot) {
          const int j = min(lane + 64 * s, ncols - 1);  // lanes past the last column recompute it (not used)
          const float4 v = ks[hh][j];
#pragma unroll
          for (int rr = 0; rr < kRowsPerWave; ++rr) {
            acc[rr][s] = fmaf(q[rr][0], v.x, acc[rr][s]);
            acc[rr][s] = fmaf(q[rr][1], v.y, acc[rr][s]);
            acc[rr][s] = fmaf(q[rr][2], v.z, acc[rr][s]);
            acc[rr][s] = fmaf(q[rr][3], v.w, acc[rr][s]);
          }
        }
      }
    }
  }

  // ---- selection of the wave's rows, from the registers
  const TpdPlan plan = wave_plan(n, a.rho_num, a.rho_den, a.mu_num, a.mu_den, lane);
  float bm[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) bm[s] = (s < wslot) ? a.beta * Mg[min(lane + 64 * s, ncols - 1)] : 0.f;
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int i = i0 + rbase + rr;
    if (i >= n) break;
    const int64_t row = (int64_t)h * a.NB + cb + i;
    const int k = (int)tpd_row_budget(plan, i);
    const int rslot = i / 64 + 1;
    uint32_t key[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int j = lane + 64 * s;
      key[s] = (s < rslot && j <= i) ? ord_key(fmaf(acc[rr][s], a.inv_sqrt_d, bm[s])) : 0u;
    }
    select_row<NS>(key, rslot, k, lane, a.mask + row * a.mask_words, a.mask_words);
    if (lane == 0) a.counts[row] = k;
  }
}

template <int NS>
void launch_ns(const ScoreTopkArgs& a, int max_n, int num_reqs, hipStream_t s) {
  const int rows = (max_n + kRows - 1) / kRows;
  if ((a.hq / a.hkv) % 2 == 0) {  // two query heads of a group per workgroup
    dim3 grid((unsigned)(a.hq / 2), (unsigned)rows, (unsigned)num_reqs);
    hipLaunchKernelGGL((score_topk_kernel<NS, 2>), grid, dim3(2 * kWavesPerHead * 64), 0, s, a);
  } else {
    dim3 grid((unsigned)a.hq, (unsigned)rows, (unsigned)num_reqs);
    hipLaunchKernelGGL((score_topk_kernel<NS, 1>), grid, dim3(kWavesPerHead * 64), 0, s, a);
  }
}

}  // namespace

hipError_t launch_score_topk(const ScoreTopkArgs& a, int max_n, int num_reqs, hipStream_t s) {
  if (max_n <= 64) launch_ns<1>(a, max_n, num_reqs, s);
  else if (max_n <= 128) launch_ns<2>(a, max_n, num_reqs, s);
  else if (max_n <= 256) launch_ns<4>(a, max_n, num_reqs, s);
  else if (max_n <= 512) launch_ns<8>(a, max_n, num_reqs, s);
  else if (max_n <= 1024) launch_ns<16>(a, max_n, num_reqs, s);
  else launch_ns<32>(a, max_n, num_reqs, s);
  return hipGetLastError();
}

}  // namespace stem
