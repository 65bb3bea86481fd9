// Stage 3 kernel: block-sparse causal flash attention over a compacted list of selected KV blocks.
//
// Source: "从Stem稀疏注意力看大模型推理的架构取舍", section "HPC-BSA：跳块零开销的秘密": for each query block the
// kernel keeps the block-mask row on chip, builds the list of KV blocks to compute, and the inner loop walks
// only that list -- the sparsity decision is taken out of the loop and the loop body is the dense one;
// skipped blocks are equivalent to -inf scores.  Fixed block size (section "答案不在算法里") makes that
// possible.  The same section's paged-KV paragraph: K/V may live in fixed-size pages behind a page table.
//
// gfx950 design (one workgroup = one (query head h, query block i), B = 32 * NW query rows):
//  * list: wave 0 compacts the mask row (bits j <= i) into an ascending uint16 list in LDS with a popcount
//    prefix scan; the diagonal block, when selected, is last.  Dense mode (no mask) walks j = 0..i.
//  * each selected block is processed as B/64 sub-tiles of 64 keys, double-buffered in LDS: K row-major
//    [64][D+pad], V transposed [D][64+pad].  Global loads for sub-tile u+1 are issued into registers before
//    sub-tile u is computed and written to the other LDS buffer afterwards (one barrier per sub-tile).
//  * S^T = K Q^T on MFMA (v_mfma_f32_32x32x16_bf16 for bf16/fp8 inputs, v_mfma_f32_32x32x2_f32 for fp32):
//    the accumulator gives each lane one query column, so the running max, the exponentials (exp2 with the
//    scale and log2(e) folded into one multiply) and the O^T rescale are per-lane scalar work; only the
//    row max needs one exchange with the partner lane (l ^ 32).
//  * O^T = V^T P^T on MFMA; P^T comes straight from the S^T registers (rounded to bf16).  The key order
//    inside each 16-key group is permuted when V is written to LDS so that the V^T operand of every MFMA
//    is one contiguous 16-byte LDS read.
//  * the causal mask is applied only on the diagonal block; waves whose rows all precede a diagonal
//    sub-tile skip it.  Padding rows of a ragged last block are computed and not stored.
//  * fp8 (OCP e4m3fn) inputs are decoded to bf16 while being staged (e4m3 values are exact in bf16); the
//    per-head scales multiply the logits (q_scale * k_scale) and the output (v_scale).
//  * work order: workgroup ids are remapped so that consecutive ids round-robin over the 8 XCDs while each
//    XCD walks one contiguous KV-head-major range (its L2 then serves the query heads of a group), with the
//    longest rows (largest block index) first.
// Bound: MFMA (effective 4 * d * visible query-key pairs).
#include <type_traits>

#include "stem_internal.h"

namespace stem {

namespace {

constexpr int KT = 64;           // keys per sub-tile
constexpr int kMaxList = 2048;   // blocks per request supported by the LDS list

template <int D, int EB>
struct Cfg {
  static constexpr bool F32 = (EB == 4);
  using lds_t = std::conditional_t<F32, float, uint16_t>;
  static constexpr int KS = D + (F32 ? 4 : 8);   // K row stride (elements)
  static constexpr int VS = KT + (F32 ? 4 : 8);  // V^T row stride (elements)
  static constexpr int K_ELEMS = KT * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int EPC = F32 ? 4 : 8;        // elements per staged chunk (one LDS vector write)
  static constexpr int K_CHUNKS = KT * D / EPC;  // chunks per K sub-tile
  static constexpr int V_TASKS = (KT / 4) * (D / EPC);  // (4 keys x EPC dims) per V task
};

// Position of key kk (0..63) of a sub-tile inside a V^T row: swap the middle two quads of every 16-key
// group so lane half h's keys {4h..4h+3, 8+4h..8+4h+3} are contiguous (bf16 path only).
__device__ __forceinline__ int vt_pos(int kk) {
  const int qd = (kk >> 2) & 3;
  const int sq = (qd == 1) ? 2 : (qd == 2 ? 1 : qd);
  return (kk & ~15) | (sq << 2) | (kk & 3);
}

// Raw global data of one chunk: 16 bytes (bf16 / f32) or 8 bytes (fp8).
template <int EB>
struct RawChunk {
  using type = std::conditional_t<EB == 1, uint2, uint4>;
};

template <int EB>
__device__ __forceinline__ typename RawChunk<EB>::type load_chunk(const void* base, int64_t elem_off) {
  using T = typename RawChunk<EB>::type;
  return *(const T*)((const uint8_t*)base + elem_off * EB);
}

// Convert one raw chunk to the LDS representation: 8 bf16 (as uint4) or 4 floats (as uint4).
template <int EB>
__device__ __forceinline__ uint4 chunk_to_lds(typename RawChunk<EB>::type w) {
  if constexpr (EB == 1) {
    float x[8];
    fp8x4_to_f32(w.x, x);
    fp8x4_to_f32(w.y, x + 4);
    return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                      pack_bf16x2(x[6], x[7]));
  } else {
    return w;
  }
}

template <int EB>
__device__ __forceinline__ typename RawChunk<EB>::type zero_chunk() {
  if constexpr (EB == 1) return make_uint2(0u, 0u);
  else return make_uint4(0u, 0u, 0u, 0u);
}

// Two workgroups per CU are asked of the register allocator only where they fit (d = 64, 16-bit K/V);
// the other instances need more registers than that allows.
template <int D, int EB>
constexpr int kMinBlocks = (D == 64 && EB != 4) ? 2 : 1;

template <int D, int EB, int NW, bool MASKED>
__global__ __launch_bounds__(NW * 64, (kMinBlocks<D, EB>)) void bsa_kernel(BsaArgs a) {
  using C = Cfg<D, EB>;
  using lds_t = typename C::lds_t;
  using raw_t = typename RawChunk<EB>::type;
  constexpr int NT = NW * 64;
  constexpr int B = NW * 32;  // query rows per block == block size
  constexpr int SPB = B / KT; // sub-tiles per block
  constexpr int KCH = (C::K_CHUNKS + NT - 1) / NT;
  constexpr int VTK = (C::V_TASKS + NT - 1) / NT;

  __shared__ __align__(16) lds_t smem[2 * C::STAGE];
  __shared__ uint16_t list[MASKED ? kMaxList : 1];
  __shared__ int list_len;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // ---- work item: (query head h, global block ib)
  const int grp = a.hq / a.hkv;
  int64_t logical = blockIdx.x;
  if (a.xcd_remap) {
    const int64_t per = (int64_t)gridDim.x / 8;
    logical = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  }
  const int64_t per_g = a.NB * grp;
  const int g = (int)(logical / per_g);
  const int64_t rem = logical % per_g;
  const int64_t ib = a.NB - 1 - rem / grp;
  const int h = g * grp + (int)(rem % grp);

  const int r = find_request(a.rt, (int)ib);
  const int i = (int)ib - a.rt.cu_blocks[r];
  const int tb = a.rt.cu_seqlens[r];
  const int L = a.rt.cu_seqlens[r + 1] - tb;

  // ---- compacted list of selected KV blocks
  int nsel;
  if constexpr (MASKED) {
    if (wave == 0) {
      const uint32_t* mrow = a.mask + ((int64_t)h * a.NB + ib) * a.mask_words;
      const int nwords = (i >> 5) + 1;
      int base = 0;
      for (int w0 = 0; w0 < nwords; w0 += 64) {
        const int w = w0 + lane;
        uint32_t word = 0;
        if (w < nwords) {
          word = mrow[w];
          if (w == nwords - 1) {
            const int nb = (i & 31) + 1;
            word &= (nb == 32) ? 0xFFFFFFFFu : ((1u << nb) - 1u);
          }
        }
        const int c = __popc(word);
        int incl = c;
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_up(incl, o, 64);
          if (lane >= o) incl += t;
        }
        int pos = base + incl - c;
        while (word) {
          const int bit = __ffs(word) - 1;
          list[pos++] = (uint16_t)(w * 32 + bit);
          word &= word - 1;
        }
        base += __shfl(incl, 63, 64);
      }
      if (lane == 0) list_len = base;
    }
    __syncthreads();
    nsel = list_len;
  } else {
    nsel = i + 1;
  }
  const int nsub = nsel * SPB;

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers for the whole loop
  const int qr = wave * 32 + l32;  // query row inside the block
  const int qpos = i * B + qr;     // request-relative token position
  const bool qvalid = qpos < L;
  constexpr int NQF = C::F32 ? D / 2 : D / 16;
  using qfrag_t = std::conditional_t<C::F32, float, bf16x8>;
  qfrag_t qf[NQF];
  {
    const int64_t qoff = ((int64_t)(tb + qpos) * a.hq + h) * D;
    if constexpr (C::F32) {
      const float* qp = (const float*)a.q + qoff;
#pragma unroll
      for (int kk = 0; kk < NQF; ++kk) qf[kk] = qvalid ? qp[2 * kk + half] : 0.f;
    } else if constexpr (EB == 2) {
      const uint16_t* qp = (const uint16_t*)a.q + qoff;
#pragma unroll
      for (int kk = 0; kk < NQF; ++kk) {
        uint4 w = qvalid ? *(const uint4*)(qp + 16 * kk + 8 * half) : make_uint4(0u, 0u, 0u, 0u);
        qf[kk] = __builtin_bit_cast(bf16x8, w);
      }
    } else {
      const uint8_t* qp = (const uint8_t*)a.q + qoff;
#pragma unroll
      for (int kk = 0; kk < NQF; ++kk) {
        uint2 w = qvalid ? *(const uint2*)(qp + 16 * kk + 8 * half) : make_uint2(0u, 0u);
        qf[kk] = __builtin_bit_cast(bf16x8, chunk_to_lds<1>(w));
      }
    }
  }
  float scale_log2 = a.scale_log2;
  float out_scale = 1.f;
  if constexpr (EB == 1) {
    scale_log2 *= a.q_scale[h] * a.k_scale[g];
    out_scale = a.v_scale[g];
  }

  // ---- staging of one 64-key sub-tile
  raw_t kreg[KCH];
  raw_t vreg[VTK][4];
  auto sub_key0 = [&](int u) -> int {
    const int j = MASKED ? (int)list[u / SPB] : u / SPB;
    return j * B + (u % SPB) * KT;
  };
  auto load_tile = [&](int u) {
    const int kp0 = sub_key0(u);
#pragma unroll
    for (int m = 0; m < KCH; ++m) {
      const int c = tid + NT * m;
      kreg[m] = zero_chunk<EB>();
      if (c < C::K_CHUNKS) {
        const int kr = c / (D / C::EPC);
        const int cc = c % (D / C::EPC);
        const int kp = kp0 + kr;
        if (kp < L) kreg[m] = load_chunk<EB>(a.k, a.kv.row(r, tb, kp, g) + cc * C::EPC);
      }
    }
#pragma unroll
    for (int m = 0; m < VTK; ++m) {
      const int tk = tid + NT * m;
#pragma unroll
      for (int e = 0; e < 4; ++e) vreg[m][e] = zero_chunk<EB>();
      if (tk < C::V_TASKS) {
        const int kq = tk % (KT / 4);
        const int dc = tk / (KT / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kp = kp0 + 4 * kq + e;
          if (kp < L) vreg[m][e] = load_chunk<EB>(a.v, a.kv.row(r, tb, kp, g) + dc * C::EPC);
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
    lds_t* Ks = smem + buf * C::STAGE;
    lds_t* Vt = Ks + C::K_ELEMS;
#pragma unroll
    for (int m = 0; m < KCH; ++m) {
      const int c = tid + NT * m;
      if (c < C::K_CHUNKS) {
        const int kr = c / (D / C::EPC);
        const int cc = c % (D / C::EPC);
        *(uint4*)(Ks + kr * C::KS + cc * C::EPC) = chunk_to_lds<EB>(kreg[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < VTK; ++m) {
      const int tk = tid + NT * m;
      if (tk < C::V_TASKS) {
        const int kq = tk % (KT / 4);
        const int dc = tk / (KT / 4);
        if constexpr (C::F32) {
          // 4 keys x 4 dims: write V^T[d][4kq .. 4kq+3] as one float4 per dim
          uint4 w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = vreg[m][e];
          const uint32_t* u0 = (const uint32_t*)&w[0];
          const uint32_t* u1 = (const uint32_t*)&w[1];
          const uint32_t* u2 = (const uint32_t*)&w[2];
          const uint32_t* u3 = (const uint32_t*)&w[3];
#pragma unroll
          for (int x = 0; x < 4; ++x)
            *(uint4*)(Vt + (dc * 4 + x) * C::VS + 4 * kq) = make_uint4(u0[x], u1[x], u2[x], u3[x]);
        } else {
          // 4 keys x 8 dims: write V^T[d][pos(4kq) .. +3] (4 bf16 = 8 bytes) per dim
          uint4 w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = chunk_to_lds<EB>(vreg[m][e]);
          const int pos = vt_pos(4 * kq);
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const uint32_t s = (x & 1) ? 16 : 0;
            const int wd = x >> 1;
            const uint32_t k0 = (((const uint32_t*)&w[0])[wd] >> s) & 0xFFFFu;
            const uint32_t k1 = (((const uint32_t*)&w[1])[wd] >> s) & 0xFFFFu;
            const uint32_t k2 = (((const uint32_t*)&w[2])[wd] >> s) & 0xFFFFu;
            const uint32_t k3 = (((const uint32_t*)&w[3])[wd] >> s) & 0xFFFFu;
            *(uint2*)(Vt + (dc * 8 + x) * C::VS + pos) = make_uint2(k0 | (k1 << 16), k2 | (k3 << 16));
          }
        }
      }
    }
  };

  // ---- running softmax state (log2 domain); O^T accumulators, lane = query column
  constexpr int NDT = D / 32;
  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int x = 0; x < 16; ++x) o[dt][x] = 0.f;
  float m_run = -INFINITY;
  float l_part = 0.f;  // sum of p over this lane's keys (partner lane holds the other half)

  if (nsub > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int u = 0; u < nsub; ++u) {
    const bool more = u + 1 < nsub;
    if (more) load_tile(u + 1);
    const int kp0 = sub_key0(u);
    const bool diag = (kp0 / B) == i;
    const bool skip = diag && (kp0 > i * B + wave * 32 + 31);
    if (!skip) {
      const lds_t* Ks = smem + (u & 1) * C::STAGE;
      const lds_t* Vt = Ks + C::K_ELEMS;
      // S^T tiles: keys [32t, 32t+32) x the wave's 32 queries
      f32x16 s[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int x = 0; x < 16; ++x) s[t][x] = 0.f;
      if constexpr (C::F32) {
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const float av = Ks[(32 * t + l32) * C::KS + 2 * kk + half];
            s[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, qf[kk], s[t], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const bf16x8 av = *(const bf16x8*)(Ks + (32 * t + l32) * C::KS + 16 * kk + 8 * half);
            s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[kk], s[t], 0, 0, 0);
          }
        }
      }
      // scale, causal mask on the diagonal, row max
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          float v = s[t][x] * scale_log2;
          if (diag) {
            const int kp = kp0 + 32 * t + 8 * (x >> 2) + 4 * half + (x & 3);
            if (kp > qpos) v = -INFINITY;
          }
          s[t][x] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const float p = exp2f(s[t][x] - m_use);
          s[t][x] = p;
          psum += p;
        }
      l_part = l_part * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int x = 0; x < 16; ++x) o[dt][x] *= alpha;
      // O^T += V^T P^T
      if constexpr (C::F32) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int kk = 32 * t + 8 * (x >> 2) + 4 * half + (x & 3);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
              const float av = Vt[(32 * dt + l32) * C::VS + kk];
              o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, s[t][x], o[dt], 0, 0, 0);
            }
          }
      } else {
#pragma unroll
        for (int mm = 0; mm < KT / 16; ++mm) {
          const int t = mm >> 1, x0 = 8 * (mm & 1);
          uint4 pw = make_uint4(pack_bf16x2(s[t][x0], s[t][x0 + 1]), pack_bf16x2(s[t][x0 + 2], s[t][x0 + 3]),
                                pack_bf16x2(s[t][x0 + 4], s[t][x0 + 5]), pack_bf16x2(s[t][x0 + 6], s[t][x0 + 7]));
          const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const bf16x8 av = *(const bf16x8*)(Vt + (32 * dt + l32) * C::VS + 16 * mm + 8 * half);
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf, o[dt], 0, 0, 0);
          }
        }
      }
    }
    if (more) store_tile((u + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue
  const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
  if (!qvalid) return;
  const float inv = (l_tot > 0.f) ? out_scale / l_tot : 0.f;
  const int64_t ooff = ((int64_t)(tb + qpos) * a.hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * dt + 8 * rq + 4 * half;
      const float v0 = o[dt][4 * rq] * inv, v1 = o[dt][4 * rq + 1] * inv;
      const float v2 = o[dt][4 * rq + 2] * inv, v3 = o[dt][4 * rq + 3] * inv;
      if constexpr (C::F32) {
        *(float4*)((float*)a.out + ooff + d0) = make_float4(v0, v1, v2, v3);
      } else {
        *(uint2*)((uint16_t*)a.out + ooff + d0) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
      }
    }
  if (a.lse != nullptr && half == 0)
    a.lse[(int64_t)h * a.tokens + tb + qpos] =
        (l_tot > 0.f) ? (m_run + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
}

template <int D, int EB, int NW>
hipError_t launch3(const BsaArgs& a, bool masked, hipStream_t s) {
  dim3 grid((unsigned)(a.hq * a.NB));
  dim3 block(NW * 64);
  if (masked) hipLaunchKernelGGL((bsa_kernel<D, EB, NW, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((bsa_kernel<D, EB, NW, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int EB>
hipError_t launch2(const BsaArgs& a, int head_dim, bool masked, hipStream_t s) {
  if (head_dim == 64) return a.B == 64 ? launch3<64, EB, 2>(a, masked, s) : launch3<64, EB, 4>(a, masked, s);
  return a.B == 64 ? launch3<128, EB, 2>(a, masked, s) : launch3<128, EB, 4>(a, masked, s);
}

}  // namespace

hipError_t launch_bsa(const BsaArgs& a, int dtype, int head_dim, bool /*paged*/, bool masked, hipStream_t s) {
  if (bsa_bf16_supported(dtype, head_dim, a.B)) return launch_bsa_bf16(a, masked, s);
  if (bsa_fp8_supported(dtype, head_dim, a.B)) return launch_bsa_fp8(a, masked, s);
  if (dtype == STEM_F32) return launch2<4>(a, head_dim, masked, s);
  if (dtype == STEM_BF16) return launch2<2>(a, head_dim, masked, s);
  return launch2<1>(a, head_dim, masked, s);
}

}  // namespace stem
