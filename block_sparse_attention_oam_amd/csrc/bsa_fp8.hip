// Block-sparse causal flash attention, fp8 (OCP e4m3fn) Q/K/V with per-head scales, head_dim 128,
// block 128: the W8A8-FP8 production layer.
//
// Source: "从Stem稀疏注意力看大模型推理的架构取舍", section "HPC-BSA：跳块零开销的秘密" (per query block: the mask row
// on chip, the list of KV blocks, the dense inner loop over the list only; skipped blocks act as -inf
// scores; paged KV) and section "答案不在算法里" (fixed block size; validation on a W8A8-FP8 model).
//
// Same work decomposition and softmax as the bf16 kernel (bsa_bf16.hip), including, when the kernel converts
// V itself and the group size is even, two query heads of a KV group per 8-wave workgroup (HEADS = 2):
//  * S^T = K Q^T runs on the fp8 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales, twice the
//    bf16 rate) on the e4m3 codes: exact products, fp32 accumulation; the logits are scaled by
//    q_scale[h] * k_scale[g] / sqrt(d) inside the exp2 argument.  K sub-tiles (64 keys x 128 bytes) go
//    global -> LDS with buffer loads that write LDS (scalar sub-tile base, fixed per-lane offsets; rows past
//    the request's end read as zeros) into a swizzled tile (slot ^ ((row >> 1) & 7)); each lane reads its
//    32-byte operand with two ds_read_b128.  Small pages look up one page per row.
//  * O^T = V^T P^T stays on the bf16 matrix cores with P in bf16: rounding P to e4m3 (3 mantissa bits)
//    misses the fp8 output tolerance on rows with few keys.  V reaches LDS as bf16, in the same swizzled
//    tile the bf16 kernel reads with ds_read_b64_tr_b16, in one of two ways:
//      VB16 = false: the kernel converts each sub-tile of V codes while staging it (global -> registers ->
//        v_cvt_scalef32_pk_bf16_fp8 -> LDS, each thread 1/(256 HEADS) of the tile, one sub-tile ahead);
//      VB16 = true: V was expanded to bf16 once, before the launch (expand_fp8_kernel: exact, every e4m3
//        value is a bf16 value), and sub-tiles go global -> LDS with buffer loads that write LDS, as K
//        does: no conversion and no LDS store per visit.  This form runs one query head per 4-wave
//        workgroup and three workgroups per CU (164 VGPRs, 52 KB of LDS each): the waves of three
//        independent workgroups overlap their matrix and vector phases better than two heads sharing
//        each tile (5.8% faster on the W8A8 128K layer).
//    Both give the same bf16 tile, so the outputs are bit-identical.
//  * softmax without a per-tile row max: the reference is set from a row's first visible keys and moves
//    only when a tile's sum of P exceeds 2^32 (the tile is then recomputed from K, still in LDS); the row
//    sum adds the rounded P pairs (v_dot2_f32_bf16).
//  * v_scale[g] multiplies the output at the end.
#include "stem_internal.h"

namespace stem {

namespace {

constexpr int D = 128;
constexpr int B = 128;
constexpr int KT = 64;
constexpr int KTILE = KT * D;      // bytes per K sub-tile (fp8)
constexpr int VTILE = KT * D * 2;  // bytes per V sub-tile (converted to bf16)
constexpr int kMaxList = 2048;
// List entries: block index in the low bits, one selection bit per head of the workgroup.
constexpr uint32_t kBlockBits = 0x3FFF;
constexpr uint32_t kSelFirst = 0x4000;
constexpr uint32_t kSelSecond = 0x8000;
constexpr float kNoReference = -1e29f;
constexpr float kOverflow = 4294967296.0f;
// Buffer resource word 3 for raw (untyped, stride 0) buffer loads on gfx9-family parts.
constexpr int kBufDword3 = 0x00020000;

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Two e4m3fn codes (the low or high 16 bits of w) -> two bf16 (exact).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// PAGE: 0 contiguous K/V, 1 pages of a multiple of 64 tokens (one page per sub-tile), 2 smaller pages.
// VB16: a.v holds V expanded to bf16 (same layout, 2-byte elements) instead of the e4m3 codes.
template <int PAGE, bool MASKED, int HEADS, bool VB16>
__global__ __launch_bounds__(256 * HEADS, (HEADS == 1 && VB16) ? 3 : 2 / HEADS) void bsa_fp8_kernel(BsaArgs a) {
  constexpr int NT = 256 * HEADS;
  constexpr int KPARTS = 2 / HEADS;    // 1 KB K loads per wave per sub-tile
  constexpr int VPARTS = 4 / HEADS;    // 1 KB bf16 V loads per wave per sub-tile (VB16)
  constexpr int VCODES = KT * D / NT;  // V codes each thread stages per sub-tile (32 or 16)
  constexpr int VTPR = D / VCODES;     // threads per V row
  constexpr int VCH = VCODES / 8;      // 16-byte bf16 chunks each thread stores
  __shared__ __align__(1024) uint8_t kbuf0[KTILE], kbuf1[KTILE], vbuf0[VTILE], vbuf1[VTILE];
  __shared__ uint16_t list[MASKED ? kMaxList : 1];
  __shared__ int list_len;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int hsel = HEADS == 2 ? wave >> 2 : 0;  // head of the workgroup this wave serves
  const int wq = HEADS == 2 ? wave & 3 : wave;   // 32-row slice of the query block
  const uint32_t mine = hsel ? kSelSecond : kSelFirst;

  // ---- work item (XCD-aware, KV-head-major, longest rows first); HEADS query heads of one KV group
  const int grp = a.hq / a.hkv;
  const int hgroups = grp / HEADS;
  int64_t logical = blockIdx.x;
  if (a.xcd_remap) {
    const int64_t per = (int64_t)gridDim.x / 8;
    logical = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  }
  const int64_t per_g = a.NB * hgroups;
  const int g = (int)(logical / per_g);
  const int64_t rem = logical % per_g;
  const int64_t ib = a.NB - 1 - rem / hgroups;
  const int h0 = g * grp + HEADS * (int)(rem % hgroups);
  const int h = h0 + hsel;
  const int r = find_request(a.rt, (int)ib);
  const int i = (int)ib - a.rt.cu_blocks[r];
  const int tb = a.rt.cu_seqlens[r];
  const int L = a.rt.cu_seqlens[r + 1] - tb;
  auto mask_row = [&](int t) { return a.mask + ((int64_t)(h0 + t) * a.NB + ib) * a.mask_words; };

  // ---- list of selected blocks (union over the workgroup's heads, one selection bit per head)
  int nsel;
  if constexpr (MASKED) {
    if (wave == 0) {
      const int nwords = (i >> 5) + 1;
      int base = 0;
      for (int w0 = 0; w0 < nwords; w0 += 64) {
        const int w = w0 + lane;
        uint32_t wa = 0, wb = 0;
        if (w < nwords) {
          const uint32_t keep = (w == nwords - 1 && (i & 31) != 31) ? ((1u << ((i & 31) + 1)) - 1u) : 0xFFFFFFFFu;
          wa = mask_row(0)[w] & keep;
          if (HEADS == 2) wb = mask_row(1)[w] & keep;
        }
        uint32_t word = wa | wb;
        const int c = __popc(word);
        int incl = c;
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_up(incl, o, 64);
          if (lane >= o) incl += t;
        }
        int pos = base + incl - c;
        while (word) {
          const int bit = __ffs(word) - 1;
          const uint32_t sel = (((wa >> bit) & 1u) ? kSelFirst : 0u) | (((wb >> bit) & 1u) ? kSelSecond : 0u);
          list[pos++] = (uint16_t)((uint32_t)(w * 32 + bit) | sel);
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
  const int nsub = nsel * 2;

  // ---- Q fragments (B operand of S^T): 32 bytes of dims 64kk + 32half.. per k-step
  const int qr = wq * 32 + l32;
  const int qpos = i * B + qr;
  const bool qvalid = qpos < L;
  i32x8 qf[2];
  {
    const uint8_t* qp = (const uint8_t*)a.q + ((int64_t)(tb + qpos) * a.hq + h) * D;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint4 w0 = make_uint4(0u, 0u, 0u, 0u), w1 = w0;
      if (qvalid) {
        w0 = *(const uint4*)(qp + 64 * kk + 32 * half);
        w1 = *(const uint4*)(qp + 64 * kk + 32 * half + 16);
      }
      qf[kk] = i32x8{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
    }
  }
  const float c2 = a.scale_log2 * a.q_scale[h] * a.k_scale[g];
  const float v_scale = a.v_scale[g];

  const int64_t row_stride = (int64_t)a.hkv * D;
  const uint8_t* kbase_all = (const uint8_t*)a.k;
  const uint8_t* vbase_all = (const uint8_t*)a.v;
  const int64_t head_off = (int64_t)g * D;

  auto entry = [&](int u) -> uint32_t {
    if constexpr (MASKED) return (uint32_t)list[u >> 1];
    else return (uint32_t)(u >> 1) | kSelFirst | kSelSecond;
  };
  // first key of sub-tile u; only list entries pack the block index (dense steps walk j = u/2, which may
  // exceed the list's 14 bits)
  auto sub_key0 = [&](uint32_t e, int u) -> int {
    const int j = MASKED ? (int)(e & kBlockBits) : (u >> 1);
    return j * B + (u & 1) * KT;
  };
  auto key_row_off = [&](int kp) -> int64_t {
    if (PAGE == 0) return ((int64_t)tb + kp) * row_stride + head_off;
    const int page = a.kv.page_table[(int64_t)r * a.kv.pt_stride + kp / a.kv.page_size];
    return ((int64_t)page * a.kv.page_size + (kp % a.kv.page_size)) * row_stride + head_off;
  };
  // byte offset of tile row `row` of the sub-tile starting at key kp0 (rows past the end repeat the last
  // key: they are causally masked)
  auto tile_row_off = [&](int kp0, int row) -> int64_t {
    if (PAGE != 2 && kp0 + KT <= L) return key_row_off(kp0) + (int64_t)row * row_stride;
    return key_row_off(min(kp0 + row, L - 1));
  };

  // ---- K loader: instruction m of this wave fills LDS chunk c = KPARTS*wave + m = tile rows 8c + lane/8,
  //      slot lane & 7 (16 bytes); the lane fetches the swizzled source chunk.
  // (fixed size 2: lambdas that capture arrays of template-dependent size lose their host stubs)
  int krow_ld[2], koff_ld[2];
#pragma unroll
  for (int m = 0; m < KPARTS; ++m) {
    const int row = 8 * (KPARTS * wave + m) + (lane >> 3);
    krow_ld[m] = row;
    koff_ld[m] = row * (int)row_stride + ((lane & 7) ^ ((row >> 1) & 7)) * 16;
  }
  auto issue_k = [&](int u, uint8_t* kdst) {
    const int kp0 = sub_key0(entry(u), u);
    if (kp0 >= L) return;  // a second half-block past the end of the request: nothing to load
    lds_u8* kl = (lds_u8*)kdst + wave * (KPARTS * 1024);
    if (PAGE == 0 || PAGE == 1) {
      const int nrec = min(L - kp0, KT) * (int)row_stride;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(kbase_all + key_row_off(kp0)), 0, nrec, kBufDword3);
#pragma unroll
      for (int m = 0; m < KPARTS; ++m)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, kl + m * 1024, 16, koff_ld[m], 0, 0, 0);
    } else {
#pragma unroll
      for (int m = 0; m < KPARTS; ++m) {
        const int row = krow_ld[m];
        const int kc = (lane & 7) ^ ((row >> 1) & 7);
        __builtin_amdgcn_global_load_lds((const void*)(kbase_all + tile_row_off(kp0, row) + kc * 16),
                                         kl + m * 1024, 16, 0, 0);
      }
    }
  };
  // V expanded to bf16 (VB16): instruction m of this wave fills LDS chunk c = VPARTS*wave + m = tile rows
  // 4c + lane/16 (256 bytes each), slot lane & 15, with the lane fetching source chunk slot ^ 4(row & 3):
  // the swizzled tile that store_v writes in the other mode.
  int vrow_ld[4], vchunk_ld[4], voff_ld[4];
#pragma unroll
  for (int m = 0; m < VPARTS; ++m) {
    const int row = 4 * (VPARTS * wave + m) + (lane >> 4);
    vrow_ld[m] = row;
    vchunk_ld[m] = (lane & 15) ^ (4 * (row & 3));
    voff_ld[m] = row * (int)(2 * row_stride) + vchunk_ld[m] * 16;
  }
  auto issue_v16 = [&](int u, uint8_t* vdst) {
    const int kp0 = sub_key0(entry(u), u);
    if (kp0 >= L) return;
    lds_u8* vl = (lds_u8*)vdst + wave * (VPARTS * 1024);
    if (PAGE == 0 || PAGE == 1) {
      const int nrec = min(L - kp0, KT) * (int)(2 * row_stride);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(vbase_all + 2 * key_row_off(kp0)), 0, nrec, kBufDword3);
#pragma unroll
      for (int m = 0; m < VPARTS; ++m)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, vl + m * 1024, 16, voff_ld[m], 0, 0, 0);
    } else {
#pragma unroll
      for (int m = 0; m < VPARTS; ++m)
        __builtin_amdgcn_global_load_lds(
            (const void*)(vbase_all + 2 * key_row_off(min(kp0 + vrow_ld[m], L - 1)) + vchunk_ld[m] * 16),
            vl + m * 1024, 16, 0, 0);
    }
  };
  // V: thread t loads VCODES codes of tile row t / VTPR (dims VCODES (t % VTPR) ..), converts them to bf16
  // and stores VCH 16-byte chunks c = VCH (t % VTPR) + j at slot c ^ 4(row & 3) of the bf16 tile (256-byte
  // rows), in the order (j + row) mod VCH so that one store instruction spreads over the bank groups.
  const int vrow = tid / VTPR, vq = tid % VTPR;
  uint4 vraw[2];
  auto load_v = [&](int u) {
    const uint8_t* src = vbase_all + tile_row_off(sub_key0(entry(u), u), vrow) + VCODES * vq;
    vraw[0] = *(const uint4*)src;
    if (VCODES == 32) vraw[1] = *(const uint4*)(src + 16);
  };
  auto store_v = [&](uint8_t* vdst) {
    const uint32_t w[8] = {vraw[0].x, vraw[0].y, vraw[0].z, vraw[0].w, vraw[1].x, vraw[1].y, vraw[1].z, vraw[1].w};
    lds_u8* row = (lds_u8*)vdst + vrow * 256;
#pragma unroll
    for (int jj = 0; jj < VCH; ++jj) {
      const int j = (jj + vrow) & (VCH - 1);  // chunk j holds dims VCODES vq + 8j .. +8 = codes w[2j], w[2j+1]
      const i32x4 c = {(int)fp8x2_to_bf16x2<false>(w[2 * j]), (int)fp8x2_to_bf16x2<true>(w[2 * j]),
                       (int)fp8x2_to_bf16x2<false>(w[2 * j + 1]), (int)fp8x2_to_bf16x2<true>(w[2 * j + 1])};
      const int chunk = VCH * vq + j;
      *(__attribute__((address_space(3))) i32x4*)(row + 16 * (chunk ^ (4 * (vrow & 3)))) = c;
    }
  };

  // ---- operand read offsets (bytes inside a tile)
  // K: row kr = 32t + l32; 16-byte slots 4kk + 2half (+1) at slot ^ ((kr >> 1) & 7); (kr >> 1) & 7 = (l32 >> 1) & 7.
  const uint32_t krow = l32 * 128;
  const int kx = (l32 >> 1) & 7;
  // V^T (bf16 tile) via ds_read_b64_tr_b16, as in the bf16 kernel.
  uint32_t voffs[4];
  {
    const int G = lane >> 4, s16 = lane & 15, rr = s16 >> 2, c = s16 & 3;
    const int row0 = 4 * (G >> 1) + rr;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int chunk = 4 * dt + 2 * (G & 1) + (c >> 1);
      voffs[dt] = row0 * 256 + 16 * (chunk ^ (4 * rr)) + 8 * (c & 1);
    }
  }

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int x = 0; x < 16; ++x) o[dt][x] = 0.f;
  float m_run = -1e30f;  // reference max (log2 units of the scaled logits)
  float l_part = 0.f;

  // Step u: K(u) (DMA) and V(u) (converted) are in LDS; K(u+1) and V(u+1) start loading into the other
  // buffers; V(u+1) is converted and stored after the compute, before the next barrier.
  auto step = [&](int u, const uint8_t* kcur, const uint8_t* vcur, uint8_t* knext, uint8_t* vnext) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const bool more = u + 1 < nsub;
    if (more) {
      if constexpr (VB16) issue_v16(u + 1, vnext);
      else load_v(u + 1);
      issue_k(u + 1, knext);
    }
    const uint32_t e = entry(u);
    const int kp0 = sub_key0(e, u);
    const bool diag = (kp0 / B) == i;
    // nothing to compute: the sub-tile starts past the request's end, or (diagonal block) every key is
    // after the wave's rows, or the wave's head did not select the block
    const bool idle = kp0 >= L || (diag && kp0 > i * B + wq * 32 + 31) || !(e & mine);
    if (!idle) {
      const lds_u8* Kt = (const lds_u8*)kcur;
      const lds_u8* Vt = (const lds_u8*)vcur;
      f32x16 s0, s1;
      auto scores = [&]() {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          s0[x] = 0.f;
          s1[x] = 0.f;
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int sa = 4 * kk + 2 * half;
          const uint32_t o0 = krow + 16 * (sa ^ kx), o1 = krow + 16 * ((sa + 1) ^ kx);
          const i32x4 a00 = *(const __attribute__((address_space(3))) i32x4*)(Kt + o0);
          const i32x4 a01 = *(const __attribute__((address_space(3))) i32x4*)(Kt + o1);
          const i32x4 a10 = *(const __attribute__((address_space(3))) i32x4*)(Kt + o0 + 32 * 128);
          const i32x4 a11 = *(const __attribute__((address_space(3))) i32x4*)(Kt + o1 + 32 * 128);
          const i32x8 f0 = {a00[0], a00[1], a00[2], a00[3], a01[0], a01[1], a01[2], a01[3]};
          const i32x8 f1 = {a10[0], a10[1], a10[2], a10[3], a11[0], a11[1], a11[2], a11[3]};
          s0 = mfma_fp8(f0, qf[kk], s0);
          s1 = mfma_fp8(f1, qf[kk], s1);
        }
        if (diag) {
          // key kp0 + 8(x/4) + 4 half + x%4 (+32 for s1) is after the query when its constant part
          // 8(x/4) + x%4 exceeds lim; lim passes through an empty asm so that the compares stay in this
          // branch (hoisted out of the retry loop they would run on every sub-tile)
          int lim = qpos - kp0 - 4 * half;
          asm volatile("" : "+v"(lim));
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int c = 8 * (x >> 2) + (x & 3);
            if (c > lim) s0[x] = -INFINITY;
            if (c + 32 > lim) s1[x] = -INFINITY;
          }
        }
      };
      // Move the reference max to this tile's max (O^T and the sum rescale by 2^(old - new), exact).
      auto rebase = [&]() {
        float mx = max3(s0[0], s0[1], s1[0]);
        mx = max3(mx, s0[2], s1[1]);
#pragma unroll
        for (int x = 3; x < 16; ++x) mx = max3(mx, s0[x], s1[x - 1]);
        mx = fmaxf(mx, s1[15]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const float m_new = fmaxf(m_run, mx * c2);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_part *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int x = 0; x < 16; ++x) o[dt][x] *= alpha;
        m_run = m_new;
      };
      uint4 pw[4];  // P rounded to bf16 pairs, the B operand of each PV k-step
      auto exp_pack = [&]() -> float {
        const float negm = -m_run;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          s0[x] = __builtin_amdgcn_exp2f(fmaf(s0[x], c2, negm));
          s1[x] = __builtin_amdgcn_exp2f(fmaf(s1[x], c2, negm));
        }
        const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          const f32x16& st = (mm < 2) ? s0 : s1;
          const int x0 = 8 * (mm & 1);
          pw[mm] = make_uint4(cvt_bf16x2(st[x0], st[x0 + 1]), cvt_bf16x2(st[x0 + 2], st[x0 + 3]),
                              cvt_bf16x2(st[x0 + 4], st[x0 + 5]), cvt_bf16x2(st[x0 + 6], st[x0 + 7]));
          ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[mm].x), ones, ps0, false);
          ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[mm].y), ones, ps1, false);
          ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[mm].z), ones, ps0, false);
          ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[mm].w), ones, ps1, false);
        }
        return ps0 + ps1;
      };
      // Rebase at the first visible keys of a row; if a tile overflows the reference, compute it again
      // with a rebase (at most once: after a rebase every P is <= 1).
      bool force = __ballot(m_run < kNoReference) != 0;
      float ps;
      for (;;) {
        asm volatile("" ::: "memory");  // keep the K reads inside the (rarely repeated) loop body
        scores();
        if (force) rebase();
        ps = exp_pack();
        if (force || __ballot(!(ps <= kOverflow)) == 0) break;
        force = true;
      }
      l_part += ps;
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pw[mm]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const lds_u8* vp = Vt + voffs[dt] + mm * 4096;
          const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)vp);
          const i16x4 v1 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vp + 2048));
          const uint2 w0 = __builtin_bit_cast(uint2, v0), w1 = __builtin_bit_cast(uint2, v1);
          const uint4 vw = make_uint4(w0.x, w0.y, w1.x, w1.y);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vw), pf, o[dt], 0, 0, 0);
        }
      }
    }
    if constexpr (!VB16)
      if (more) store_v(vnext);
  };

  if (nsub > 0) {
    if constexpr (VB16) {
      issue_v16(0, vbuf0);
      issue_k(0, kbuf0);
    } else {
      load_v(0);
      issue_k(0, kbuf0);
      store_v(vbuf0);
    }
  }
  for (int u = 0; u < nsub; u += 2) {
    step(u, kbuf0, vbuf0, kbuf1, vbuf1);
    if (u + 1 < nsub) step(u + 1, kbuf1, vbuf1, kbuf0, vbuf0);
  }

  // ---- epilogue
  const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
  if (!qvalid) return;
  const float inv = (l_tot > 0.f) ? v_scale / l_tot : 0.f;  // V (codes or their bf16 values) is unscaled
  const int64_t ooff = ((int64_t)(tb + qpos) * a.hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * dt + 8 * rq + 4 * half;
      *(uint2*)((uint16_t*)a.out + ooff + d0) =
          make_uint2(pack_bf16x2(o[dt][4 * rq] * inv, o[dt][4 * rq + 1] * inv),
                     pack_bf16x2(o[dt][4 * rq + 2] * inv, o[dt][4 * rq + 3] * inv));
    }
  if (a.lse != nullptr && half == 0)
    a.lse[(int64_t)h * a.tokens + tb + qpos] =
        (l_tot > 0.f) ? (m_run + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
}

// V codes -> bf16 (exact), 16 codes per thread.  n is a multiple of 16; src and dst are 16-byte aligned.
__global__ __launch_bounds__(256) void expand_fp8_kernel(const uint8_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                         int64_t n16) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n16) return;
  const uint4 w = ((const uint4*)src)[t];
  const uint32_t c[4] = {w.x, w.y, w.z, w.w};
  uint4 out[2];
  uint32_t* o = (uint32_t*)out;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    o[2 * x] = fp8x2_to_bf16x2<false>(c[x]);
    o[2 * x + 1] = fp8x2_to_bf16x2<true>(c[x]);
  }
  ((uint4*)dst)[2 * t] = out[0];
  ((uint4*)dst)[2 * t + 1] = out[1];
}

template <bool MASKED, int HEADS, bool VB16>
static hipError_t launch_fp8_heads(const BsaArgs& args, hipStream_t s) {
  BsaArgs a = args;
  const int64_t wgs = (int64_t)(a.hq / HEADS) * a.NB;
  a.xcd_remap = wgs % 8 == 0 ? 1 : 0;
  const dim3 grid((unsigned)wgs), block(256 * HEADS);
  const int page_mode = !a.kv.paged ? 0 : (a.kv.page_size % KT == 0 ? 1 : 2);
  if (page_mode == 0) hipLaunchKernelGGL((bsa_fp8_kernel<0, MASKED, HEADS, VB16>), grid, block, 0, s, a);
  else if (page_mode == 1) hipLaunchKernelGGL((bsa_fp8_kernel<1, MASKED, HEADS, VB16>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((bsa_fp8_kernel<2, MASKED, HEADS, VB16>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <bool VB16>
static hipError_t launch_fp8_v(const BsaArgs& a, bool masked, hipStream_t s) {
  if constexpr (VB16) {
    // expanded V: one head per workgroup, three workgroups per CU
    return masked ? launch_fp8_heads<true, 1, true>(a, s) : launch_fp8_heads<false, 1, true>(a, s);
  } else {
    // V converted per visit: two heads per workgroup when the group size is even
    const bool pair = (a.hq / a.hkv) % 2 == 0;
    if (masked) return pair ? launch_fp8_heads<true, 2, false>(a, s) : launch_fp8_heads<true, 1, false>(a, s);
    return pair ? launch_fp8_heads<false, 2, false>(a, s) : launch_fp8_heads<false, 1, false>(a, s);
  }
}

}  // namespace

bool bsa_fp8_supported(int dtype, int head_dim, int block) {
  return dtype == STEM_FP8_E4M3 && head_dim == D && block == B;
}

hipError_t launch_bsa_fp8(const BsaArgs& a, bool masked, hipStream_t s) { return launch_fp8_v<false>(a, masked, s); }

hipError_t launch_expand_fp8(const void* v_codes, void* v_bf16, int64_t n, hipStream_t s) {
  const int64_t n16 = n / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(expand_fp8_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                     (const uint8_t*)v_codes, (uint16_t*)v_bf16, n16);
  return hipGetLastError();
}

hipError_t launch_bsa_fp8_vb16(const BsaArgs& a, bool masked, hipStream_t s) {
  return launch_fp8_v<true>(a, masked, s);
}

}  // namespace stem
