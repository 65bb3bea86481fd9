// Stage 1 kernels: block pooling of Q/K/V and the OAM scoring GEMM.
//
// Source: "从Stem稀疏注意力看大模型推理的架构取舍", sections "OAM：价值评估" (score = routing relevance
// QK^T + beta * log||V_j||_2) and "HPC-Stem：评估选块，快几十倍" (the additive score lets compact per-block
// Q and K representations replace the token-level product, so all block scores come from one GEMM).
//
// pool_kernel   HBM-bound streaming reduction.  One workgroup owns one block (B tokens) and a 256-lane
//               slice of the token row (16 bytes per lane per token, so every load is a coalesced 16-byte
//               vector).  Q and K are summed in fp32 and divided by the number of valid tokens; V rows
//               give ln||v||_2 per (token, head) through a shuffle reduction over the lanes of the head,
//               averaged over the block.  Algorithmic bytes: one read of Q, K and V plus the fp32 outputs.
// score_kernel  S = qbar kbar^T / sqrt(d) + beta M for the causal tile pairs of each request, fp32 FMA
//               in a 64x64 register-blocked tile (4x4 per thread), d staged through LDS in chunks of 32.
#include "stem_internal.h"

namespace stem {

namespace {

constexpr int kPoolThreads = 256;

// Decode one 16-byte vector into N = 16/EB floats.
template <int EB>
__device__ __forceinline__ void decode16(const uint4 w, float* x) {
  if constexpr (EB == 4) {
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z);
    x[3] = __uint_as_float(w.w);
  } else if constexpr (EB == 2) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(u[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_bits_to_f32(u[i] >> 16);
    }
  } else {
    fp8x4_to_f32(w.x, x);
    fp8x4_to_f32(w.y, x + 4);
    fp8x4_to_f32(w.z, x + 8);
    fp8x4_to_f32(w.w, x + 12);
  }
}

// Sixteen bf16 values (32 bytes) -> per-head-scaled e4m3fn codes (RNE, saturated at +-448), packed.
__device__ __forceinline__ uint4 quant16(const uint4 w0, const uint4 w1, float s) {
  float x[16];
  decode16<2>(w0, x);
  decode16<2>(w1, x + 8);
  uint32_t c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(x[4 * i + e] / s, -448.f), 448.f);
    int wv = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    wv = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], wv, true);
    c[i] = (uint32_t)wv;
  }
  return make_uint4(c[0], c[1], c[2], c[3]);
}

// QUANT: the inputs are bf16; each lane reads the 16 values that an fp8 lane would, quantises them with its
// head's scale, stores the codes and pools the decoded codes exactly as the fp8 pool does.
template <int EB, bool QUANT = false>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(PoolArgs a) {
  static_assert(!QUANT || EB == 1, "quantising pool uses the fp8 lane layout");
  constexpr int EPL = 16 / EB;  // elements per lane
  const int ib = blockIdx.x;
  int job = blockIdx.y;
  int kind;  // 0 = Q mean, 1 = K mean, 2 = V log-norm mean (V jobs first: they take longest per byte)
  if (job < a.kv_chunks) {
    kind = 2;
  } else if (job < 2 * a.kv_chunks) {
    kind = 1;
    job -= a.kv_chunks;
  } else {
    kind = 0;
    job -= 2 * a.kv_chunks;
  }
  const int H = kind == 0 ? a.hq : a.hkv;
  const int d = a.d;
  const int lpr = H * d / EPL;  // lanes per token row
  const int chunk_lanes = min(lpr - job * kPoolThreads, kPoolThreads);
  const int tr = kPoolThreads / chunk_lanes;  // token rows processed in parallel
  const int tid = threadIdx.x;
  const int rs = tid / chunk_lanes;
  const int lic = tid % chunk_lanes;
  const bool active = rs < tr;

  const int r = find_request(a.rt, ib);
  const int i = ib - a.rt.cu_blocks[r];
  const int tb = a.rt.cu_seqlens[r];
  const int L = a.rt.cu_seqlens[r + 1] - tb;
  const int t0 = i * a.B;
  const int t1 = min(t0 + a.B, L);
  const int e0 = (job * kPoolThreads + lic) * EPL;  // first element of this lane in the token row
  const int head = e0 / d;
  const int dd = e0 % d;
  const int hl = d / EPL;  // lanes per head

  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float lacc = 0.f;

  const uint8_t* base;
  float vscale = 1.f;
  if (kind == 0) {
    base = (const uint8_t*)a.q;
  } else {
    base = (const uint8_t*)(kind == 1 ? a.k : a.v);
    if (EB == 1 && kind == 2) vscale = a.v_scale[head];
  }

  auto elem_off = [&](int t) -> int64_t {
    if (kind == 0) return (int64_t)(tb + t) * a.hq * d + e0;
    return a.kv.row(r, tb, t, head) + dd;
  };
  auto row_ptr = [&](int t) -> const uint4* { return (const uint4*)(base + elem_off(t) * EB); };
  float qscale = 1.f;  // quantising pool: this lane's head scale
  uint8_t* qdst = nullptr;
  if constexpr (QUANT) {
    qscale = kind == 0 ? a.q_scale[head] : (kind == 1 ? a.k_scale[head] : a.v_scale[head]);
    qdst = (uint8_t*)(kind == 0 ? a.q8 : (kind == 1 ? a.k8 : a.v8));
  }
  // 16 bytes of this lane's row t: the stored vector, or (quantising) the codes of its 32 bf16 bytes
  auto load = [&](int t) -> uint4 {
    if constexpr (QUANT) {
      const int64_t off = elem_off(t);
      const uint4* src = (const uint4*)(base + off * 2);
      const uint4 c = quant16(src[0], src[1], qscale);
      *(uint4*)(qdst + off) = c;
      return c;
    } else {
      return *row_ptr(t);
    }
  };

  if (active) {
    if (kind != 2) {
      int t = t0 + rs;
      for (; t + 3 * tr < t1; t += 4 * tr) {
        uint4 w0 = load(t), w1 = load(t + tr), w2 = load(t + 2 * tr), w3 = load(t + 3 * tr);
        float x[EPL];
        decode16<EB>(w0, x);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += x[e];
        decode16<EB>(w1, x);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += x[e];
        decode16<EB>(w2, x);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += x[e];
        decode16<EB>(w3, x);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += x[e];
      }
      for (; t < t1; t += tr) {
        float x[EPL];
        decode16<EB>(load(t), x);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += x[e];
      }
    }
  }
  if (kind == 2) {
    // All lanes of a head must take part in the shuffles: a uniform trip count per row slot; four rows per
    // trip so that four loads are in flight (the rows' log-norms are added in row order).
    for (int t = t0 + rs; t < t0 + a.B; t += 4 * tr) {
      uint4 w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tj = t + j * tr;
        w[j] = (active && tj < t1) ? load(tj) : make_uint4(0u, 0u, 0u, 0u);
      }
      float ss[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x[EPL];
        decode16<EB>(w[j], x);
        ss[j] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float y = x[e] * vscale;
          ss[j] = fmaf(y, y, ss[j]);
        }
      }
      for (int m = 1; m < hl; m <<= 1)
#pragma unroll
        for (int j = 0; j < 4; ++j) ss[j] += __shfl_xor(ss[j], m, 64);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (active && t + j * tr < t1) lacc += 0.5f * logf(ss[j]);
    }
  }

  // Combine the parallel token rows through LDS.
  __shared__ float red[kPoolThreads * 16];
  const int cnt = t1 - t0;
  if (tr > 1) {
    if (kind != 2) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[tid * EPL + e] = acc[e];
    } else {
      red[tid] = lacc;
    }
    __syncthreads();
    if (rs == 0) {
      for (int s = 1; s < tr; ++s) {
        const int src = s * chunk_lanes + lic;
        if (kind != 2) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] += red[src * EPL + e];
        } else {
          lacc += red[src];
        }
      }
    }
  }
  if (rs != 0) return;

  const float inv = 1.f / (float)cnt;
  if (kind == 2) {
    if (lic % hl == 0) a.M[(int64_t)head * a.NB + ib] = lacc * inv;
    return;
  }
  float sc = inv;
  if constexpr (EB == 1) sc *= (kind == 0 ? a.q_scale[head] : a.k_scale[head]);
  float* dst = (kind == 0 ? a.qbar : a.kbar) + ((int64_t)head * a.NB + ib) * d + dd;
#pragma unroll
  for (int e = 0; e < EPL; e += 4) {
    float4 o = make_float4(acc[e] * sc, acc[e + 1] * sc, acc[e + 2] * sc, acc[e + 3] * sc);
    *(float4*)(dst + e) = o;
  }
}

// Per-head amax of bf16 Q, K, V (for the W8A8 scales): blockIdx.y selects the tensor, blockIdx.x a range of
// 64 tokens; lanes of one head reduce by shuffles, one atomicMax per head and workgroup on the float bits
// (non-negative floats order like their bit patterns).  amax[] must start at 0.
__global__ __launch_bounds__(256) void amax_kernel(PoolArgs a, unsigned* qmax, unsigned* kmax, unsigned* vmax,
                                                   int64_t tokens) {
  const int kind = blockIdx.y;
  const int H = kind == 0 ? a.hq : a.hkv;
  const int rowlen = H * a.d;            // elements per token row
  const int lanes = rowlen / 8;          // 16-byte vectors per row
  const int hl = a.d / 8;                // lanes per head (16 or 8)
  const uint16_t* src = (const uint16_t*)(kind == 0 ? a.q : (kind == 1 ? a.k : a.v));
  unsigned* out = kind == 0 ? qmax : (kind == 1 ? kmax : vmax);
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  for (int c0 = 0; c0 < lanes; c0 += 256) {
    const int c = c0 + threadIdx.x;
    const bool ok = c < lanes;
    float m = 0.f;
    if (ok) {
      for (int64_t t = t0; t < t0 + 64 && t < tokens; ++t) {
        float x[8];
        decode16<2>(*(const uint4*)(src + t * rowlen + (int64_t)c * 8), x);
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
      }
    }
    for (int o = 1; o < hl; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (ok && (c % hl) == 0) atomicMax(out + c / hl, __float_as_uint(m));
  }
}

// amax bits -> scale = amax / 448 (1 when amax is 0), in place.
__global__ void scale_kernel(float* s, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const float amax = __uint_as_float(__float_as_uint(s[i]));
    s[i] = amax > 0.f ? amax / 448.f : 1.f;
  }
}

__global__ void zero_kernel(float* s, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) s[i] = 0.f;
}

// W8A8 quantisation alone: bf16 x [tokens][H][d] -> e4m3fn codes with the per-head scales already in
// `scale`; each thread converts 16 consecutive elements of one head (32 bytes in, 16 bytes out) with the
// same arithmetic as the quantising pool.  HBM-bound streaming.
__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* x, uint8_t* codes, const float* scale, int H,
                                                    int d, int64_t n16) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n16) return;
  const int64_t e0 = idx * 16;
  const int head = (int)((e0 / d) % H);
  const uint4* src = (const uint4*)(x + e0);
  *(uint4*)(codes + e0) = quant16(src[0], src[1], scale[head]);
}

constexpr int kTile = 64;
constexpr int kDChunk = 32;

__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  const int r = blockIdx.z;
  const int h = blockIdx.y;
  const int pidx = blockIdx.x;
  const int n = a.rt.cu_blocks[r + 1] - a.rt.cu_blocks[r];
  const int nt = (n + kTile - 1) / kTile;
  if (pidx >= nt * (nt + 1) / 2) return;
  // tile pair (I, J), J <= I, from the linear index
  int I = (int)((sqrtf(8.f * pidx + 1.f) - 1.f) * 0.5f);
  while ((I + 1) * (I + 2) / 2 <= pidx) ++I;
  while (I * (I + 1) / 2 > pidx) --I;
  const int J = pidx - I * (I + 1) / 2;
  const int g = h / (a.hq / a.hkv);
  const int64_t cb = a.rt.cu_blocks[r];
  const int d = a.d;

  __shared__ float qs[kTile][kDChunk + 1];
  __shared__ float ks[kTile][kDChunk + 1];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  float acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = 0.f;

  const float* qb = a.qbar + ((int64_t)h * a.NB + cb) * d;
  const float* kb = a.kbar + ((int64_t)g * a.NB + cb) * d;
  for (int d0 = 0; d0 < d; d0 += kDChunk) {
    // 64 rows x 32 floats per operand: 2048 floats, 8 per thread
    for (int e = tid; e < kTile * kDChunk; e += 256) {
      const int row = e / kDChunk, col = e % kDChunk;
      const int qi = I * kTile + row, kj = J * kTile + row;
      qs[row][col] = qi < n ? qb[(int64_t)qi * d + d0 + col] : 0.f;
      ks[row][col] = kj < n ? kb[(int64_t)kj * d + d0 + col] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < kDChunk; ++c) {
      float qa[4], kb4[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) qa[x] = qs[ty + 16 * x][c];
#pragma unroll
      for (int y = 0; y < 4; ++y) kb4[y] = ks[tx + 16 * y][c];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(qa[x], kb4[y], acc[x][y]);
    }
    __syncthreads();
  }
  const float* Mg = a.M + (int64_t)g * a.NB + cb;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int i = I * kTile + ty + 16 * x;
    if (i >= n) continue;
    float* row = a.scores + ((int64_t)h * a.NB + cb + i) * a.stride;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int j = J * kTile + tx + 16 * y;
      if (j <= i) row[j] = fmaf(acc[x][y], a.inv_sqrt_d, a.beta * Mg[j]);
    }
  }
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, int dtype, hipStream_t s) {
  dim3 grid((unsigned)a.NB, (unsigned)(a.q_chunks + 2 * a.kv_chunks));
  if (dtype == STEM_F32) hipLaunchKernelGGL(pool_kernel<4>, grid, dim3(kPoolThreads), 0, s, a);
  else if (dtype == STEM_BF16) hipLaunchKernelGGL(pool_kernel<2>, grid, dim3(kPoolThreads), 0, s, a);
  else hipLaunchKernelGGL(pool_kernel<1>, grid, dim3(kPoolThreads), 0, s, a);
  return hipGetLastError();
}

// Per-head scales of bf16 Q, K, V: amax over all tokens, then amax / 448 (1 for an all-zero head).
static void launch_scales(const PoolArgs& a, float* q_scale, float* k_scale, float* v_scale, int64_t tokens,
                          hipStream_t s) {
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((a.hq + 255) / 256)), dim3(256), 0, s, q_scale, a.hq);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((a.hkv + 255) / 256)), dim3(256), 0, s, k_scale, a.hkv);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((a.hkv + 255) / 256)), dim3(256), 0, s, v_scale, a.hkv);
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)((tokens + 63) / 64), 3), dim3(256), 0, s, a, (unsigned*)q_scale,
                     (unsigned*)k_scale, (unsigned*)v_scale, tokens);
  hipLaunchKernelGGL(scale_kernel, dim3((unsigned)((a.hq + 255) / 256)), dim3(256), 0, s, q_scale, a.hq);
  hipLaunchKernelGGL(scale_kernel, dim3((unsigned)((a.hkv + 255) / 256)), dim3(256), 0, s, k_scale, a.hkv);
  hipLaunchKernelGGL(scale_kernel, dim3((unsigned)((a.hkv + 255) / 256)), dim3(256), 0, s, v_scale, a.hkv);
}

hipError_t launch_quant(const PoolArgs& a, float* q_scale, float* k_scale, float* v_scale, int64_t tokens,
                        hipStream_t s) {
  launch_scales(a, q_scale, k_scale, v_scale, tokens, s);
  const int64_t nq = tokens * a.hq * a.d / 16, nkv = tokens * a.hkv * a.d / 16;
  hipLaunchKernelGGL(quant_kernel, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, s, (const uint16_t*)a.q,
                     (uint8_t*)a.q8, (const float*)q_scale, a.hq, a.d, nq);
  hipLaunchKernelGGL(quant_kernel, dim3((unsigned)((nkv + 255) / 256)), dim3(256), 0, s, (const uint16_t*)a.k,
                     (uint8_t*)a.k8, (const float*)k_scale, a.hkv, a.d, nkv);
  hipLaunchKernelGGL(quant_kernel, dim3((unsigned)((nkv + 255) / 256)), dim3(256), 0, s, (const uint16_t*)a.v,
                     (uint8_t*)a.v8, (const float*)v_scale, a.hkv, a.d, nkv);
  return hipGetLastError();
}

hipError_t launch_quant_pool(const PoolArgs& a, float* q_scale, float* k_scale, float* v_scale, int64_t tokens,
                             hipStream_t s) {
  launch_scales(a, q_scale, k_scale, v_scale, tokens, s);
  PoolArgs b = a;
  b.q_scale = q_scale;
  b.k_scale = k_scale;
  b.v_scale = v_scale;
  dim3 grid((unsigned)a.NB, (unsigned)(a.q_chunks + 2 * a.kv_chunks));
  hipLaunchKernelGGL((pool_kernel<1, true>), grid, dim3(kPoolThreads), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs& a, int max_n, int num_reqs, hipStream_t s) {
  const int nt = (max_n + kTile - 1) / kTile;
  dim3 grid((unsigned)(nt * (nt + 1) / 2), (unsigned)a.hq, (unsigned)num_reqs);
  hipLaunchKernelGGL(score_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace stem
