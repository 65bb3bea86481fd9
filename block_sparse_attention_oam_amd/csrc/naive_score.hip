// The naive, token-level form of the block metric: a comparison path, kept to measure what the pooled
// one-GEMM scoring saves.
//
// Source: "从Stem稀疏注意力看大模型推理的架构取舍", section "HPC-Stem：评估选块，快几十倍": computing the metric
// the direct way (token-level attention probabilities of sampled queries, gathered into blocks) builds
// intermediate tensors of tens of GB and is tens of times slower than scoring compact block
// representations with one GEMM.
//
// For `samples` queries per block (block i's sample s is token min(iB + s B/samples, L - 1)) and every
// query head, four kernels run one after the other, each through HBM as a straightforward implementation
// would:
//   naive_logits_kernel   logits[h][row][tau] = q_t . k_tau / sqrt(d) for every key tau < L (bf16 MFMA,
//                         fp32 out): rows x L floats per head
//   naive_softmax_kernel  in place: softmax over tau <= t, zero beyond (three passes over the row)
//   naive_mass_kernel     mass[h][row][j] = sum of the row's probabilities in key block j
//   naive_finish_kernel   S[h][i][j] = ln(mean over block i's samples of mass) + beta M[g][j], j <= i,
//                         written in stem_score's layout, so stem_tpd_topk selects from it as usual.
#include "stem_internal.h"

namespace stem {

namespace {

// position of sampled row rho (= i * samples + s) of a request of L tokens
__device__ __forceinline__ int sample_pos(int rho, int samples, int B, int L) {
  const int i = rho / samples, s = rho % samples;
  return min(i * B + s * (B / samples), L - 1);
}

// One workgroup: 32 sampled rows x 128 keys (4 waves x 32 keys), v_mfma_f32_32x32x16_bf16 with both
// operands loaded straight from global memory (lane l: row/key l % 32, dims 8 (l / 32) .. + 8 of the step).
__global__ __launch_bounds__(256) void naive_logits_kernel(NaiveArgs a, int r) {
  const int h = blockIdx.z;
  const int g = h / (a.hq / a.hkv);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int l32 = lane & 31, half = lane >> 5;
  const int tb = a.rt.cu_seqlens[r];
  const int L = a.rt.cu_seqlens[r + 1] - tb;
  const int n = a.rt.cu_blocks[r + 1] - a.rt.cu_blocks[r];
  const int R = n * a.samples;
  const int rho0 = blockIdx.y * 32;
  const int tau0 = blockIdx.x * 128 + wave * 32;
  if (tau0 >= L) return;  // whole wave past the keys (no barrier below)
  const int rho = min(rho0 + l32, R - 1);
  const int t = sample_pos(rho, a.samples, a.B, L);
  const int tau = min(tau0 + l32, L - 1);
  const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)(tb + t) * a.hq + h) * a.d + 8 * half;
  const uint16_t* kp = (const uint16_t*)a.k + ((int64_t)(tb + tau) * a.hkv + g) * a.d + 8 * half;
  f32x16 c;
#pragma unroll
  for (int x = 0; x < 16; ++x) c[x] = 0.f;
  for (int kk = 0; kk < a.d / 16; ++kk) {
    const bf16x8 qa = __builtin_bit_cast(bf16x8, *(const uint4*)(qp + 16 * kk));
    const bf16x8 kb = __builtin_bit_cast(bf16x8, *(const uint4*)(kp + 16 * kk));
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kb, c, 0, 0, 0);
  }
  // C layout: lane l holds key column l % 32 and rows 8 (x / 4) + 4 (l / 32) + x % 4
  float* buf = a.buf + (int64_t)h * a.rows_max * a.row_stride;
  const int kcol = tau0 + l32;
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const int row = rho0 + 8 * (x >> 2) + 4 * half + (x & 3);
    if (row < R && kcol < L) buf[(int64_t)row * a.row_stride + kcol] = c[x] * a.scale;
  }
}

__device__ __forceinline__ float block_reduce(float v, bool is_max, float* red) {
  for (int o = 32; o > 0; o >>= 1) {
    const float w = __shfl_xor(v, o, 64);
    v = is_max ? fmaxf(v, w) : v + w;
  }
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = red[0];
  for (int w = 1; w < 4; ++w) t = is_max ? fmaxf(t, red[w]) : t + red[w];
  return t;
}

// One workgroup per (row, head): the row's softmax over tau <= t, written in place; keys after t get 0.
__global__ __launch_bounds__(256) void naive_softmax_kernel(NaiveArgs a, int r) {
  __shared__ float red[4];
  const int rho = blockIdx.x, h = blockIdx.y;
  const int tb = a.rt.cu_seqlens[r];
  const int L = a.rt.cu_seqlens[r + 1] - tb;
  const int t = sample_pos(rho, a.samples, a.B, L);
  float* row = a.buf + ((int64_t)h * a.rows_max + rho) * a.row_stride;
  float mx = -INFINITY;
  for (int tau = threadIdx.x; tau <= t; tau += 256) mx = fmaxf(mx, row[tau]);
  mx = block_reduce(mx, true, red);
  float sum = 0.f;
  for (int tau = threadIdx.x; tau <= t; tau += 256) sum += expf(row[tau] - mx);
  sum = block_reduce(sum, false, red);
  const float inv = 1.f / sum;
  for (int tau = threadIdx.x; tau < L; tau += 256) row[tau] = tau <= t ? expf(row[tau] - mx) * inv : 0.f;
}

// One workgroup per (row, head): block sums of the row's probabilities, one wavefront per block.
__global__ __launch_bounds__(256) void naive_mass_kernel(NaiveArgs a, int r) {
  const int rho = blockIdx.x, h = blockIdx.y;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int tb = a.rt.cu_seqlens[r];
  const int L = a.rt.cu_seqlens[r + 1] - tb;
  const int n = a.rt.cu_blocks[r + 1] - a.rt.cu_blocks[r];
  const float* row = a.buf + ((int64_t)h * a.rows_max + rho) * a.row_stride;
  float* mrow = a.mass + ((int64_t)h * a.rows_max + rho) * a.mass_stride;
  for (int j = wave; j < n; j += 4) {
    float s = 0.f;
    for (int e = lane; e < a.B; e += 64) {
      const int tau = j * a.B + e;
      if (tau < L) s += row[tau];
    }
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0) mrow[j] = s;
  }
}

// One thread per (i, j <= i) entry of a score row: ln of the mean mass over block i's samples + beta M.
__global__ __launch_bounds__(256) void naive_finish_kernel(NaiveArgs a, int r) {
  const int i = blockIdx.x, h = blockIdx.y;
  const int g = h / (a.hq / a.hkv);
  const int64_t cb = a.rt.cu_blocks[r];
  const float* mbase = a.mass + ((int64_t)h * a.rows_max + (int64_t)i * a.samples) * a.mass_stride;
  float* srow = a.scores + ((int64_t)h * a.NB + cb + i) * a.stride;
  for (int j = threadIdx.x; j <= i; j += 256) {
    float s = 0.f;
    for (int k = 0; k < a.samples; ++k) s += mbase[(int64_t)k * a.mass_stride + j];
    srow[j] = logf(s / (float)a.samples) + a.beta * a.M[(int64_t)g * a.NB + cb + j];
  }
}

}  // namespace

hipError_t launch_naive(const NaiveArgs& a, const int32_t* lens, const int32_t* nblocks, int num_reqs,
                        hipStream_t s) {
  for (int r = 0; r < num_reqs; ++r) {
    const int L = lens[r];
    const int n = nblocks[r];
    if (n == 0) continue;
    const int R = n * a.samples;
    hipLaunchKernelGGL(naive_logits_kernel, dim3((unsigned)((L + 127) / 128), (unsigned)((R + 31) / 32), (unsigned)a.hq),
                       dim3(256), 0, s, a, r);
    hipLaunchKernelGGL(naive_softmax_kernel, dim3((unsigned)R, (unsigned)a.hq), dim3(256), 0, s, a, r);
    hipLaunchKernelGGL(naive_mass_kernel, dim3((unsigned)R, (unsigned)a.hq), dim3(256), 0, s, a, r);
    hipLaunchKernelGGL(naive_finish_kernel, dim3((unsigned)n, (unsigned)a.hq), dim3(256), 0, s, a, r);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace stem
