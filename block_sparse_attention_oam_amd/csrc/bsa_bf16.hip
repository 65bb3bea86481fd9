// Block-sparse causal flash attention, bf16 inputs, head_dim 128, block 128 (the main production shape).
//
// Source: "从Stem稀疏注意力看大模型推理的架构取舍", section "HPC-BSA：跳块零开销的秘密" (per query block: keep the
// mask row on chip, build the list of KV blocks, iterate only over the list with the dense inner loop;
// skipped blocks act as -inf scores; K/V may sit in pages behind a page table) and section "答案不在算法里"
// (the fixed block size is what lets the decision leave the inner loop).
//
// Same mathematics and work decomposition as the generic kernel (bsa_fwd.hip); this version is shaped for
// gfx950's issue limits, because the generic one spends ~24 VALU instructions per MFMA:
//  * K and V sub-tiles (64 keys x 128 dims, 16 KB each) go from global memory straight into LDS with
//    global_load_lds_dwordx4 (lane l of an instruction fills the l-th 16-byte slot of a 1 KB LDS chunk):
//    no staging registers, no LDS store or repacking instructions.  The loads of sub-tile u+1 are issued
//    after the barrier of sub-tile u and overlap its compute (double buffer, one barrier per sub-tile).
//  * tiles are row-major without padding (a 256-byte row spans the 64 LDS banks once); 16-byte slots are
//    XOR-swizzled by row (K: slot ^ (row & 15), V: slot ^ 4*(row & 3)), which the loading lanes apply by
//    choosing their source chunk.  A ds_read_b128 pass (16 lanes, 16 consecutive K rows, one chunk) and a
//    ds_read_b64_tr_b16 pass (32 lanes, 4 V rows x 4 chunks) then touch every bank once.
//  * S^T = K Q^T (v_mfma_f32_32x32x16_bf16): K operand = one ds_read_b128 per MFMA.  O^T = V^T P^T: the V^T
//    operand is gathered from the row-major V tile by two ds_read_b64_tr_b16 (transposing 16-bit reads),
//    in the key order that the S^T accumulator layout gives P^T, so P never moves between lanes.
//  * softmax: raw v_exp_f32 (no denormal fix-up) of one FMA that folds the scale and the reference max.
//    There is no per-tile row max: the reference is taken from the first visible keys of each row and
//    kept while a tile's sum of P stays <= 2^32 (bf16 and fp32 have the same exponent range, so P keeps
//    its relative precision at any scale); a larger sum (or inf) recomputes the tile's scores, moves
//    the reference to their max and rescales O^T and the sum exactly.  The row sum adds the rounded P
//    pairs with v_dot2_f32_bf16 (the same values PV multiplies).
//  * sub-tile loads are buffer loads (contiguous K/V, or pages of >= 64 tokens): the sub-tile's base
//    address is scalar and each lane's byte offset is fixed, so issuing a load costs no vector
//    instructions; rows past the request's end fall outside the buffer and read as zeros.  Small pages
//    look up one page per row.  The diagonal block takes a separate path with the causal mask; other
//    blocks have no per-element compares.
//  * HEADS = 2 (an even number of query heads per KV head): one workgroup of 8 waves serves the same query
//    block of two query heads of a KV group (waves 0-3 the first, 4-7 the second), so every K/V sub-tile it
//    loads feeds twice the MFMA work and each wave issues half the loads.  The list is the union of the
//    two mask rows, each entry carrying one selection bit per head; a wave skips the compute of a block its
//    head did not select (the heads of a KV group select nearly the same blocks).
#include "stem_internal.h"

namespace stem {

namespace {

constexpr int D = 128;
constexpr int B = 128;
constexpr int KT = 64;
constexpr int TILE = KT * D * 2;  // bytes per K or V sub-tile
constexpr int kMaxList = 2048;
// List entries: block index in the low bits, one selection bit per head of the workgroup.
constexpr uint32_t kBlockBits = 0x3FFF;
constexpr uint32_t kSelFirst = 0x4000;
constexpr uint32_t kSelSecond = 0x8000;
// Softmax reference point: the reference max m_run (log2 units) is set from the first visible keys of a
// row and then kept while the tile sums of P = 2^(s - m_run) stay <= 2^32 (no overflow anywhere in P,
// the row sum or O^T); a larger sum rebases to the tile's max.  P keeps bf16's relative precision at any
// scale, so no per-tile max is needed.
constexpr float kNoReference = -1e29f;
constexpr float kOverflow = 4294967296.0f;
// Buffer resource word 3 for raw (untyped, stride 0) buffer loads on gfx9-family parts.
constexpr int kBufDword3 = 0x00020000;

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;

// Two floats -> packed bf16 pair (round to nearest even) with one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// PAGE: 0 contiguous K/V, 1 pages of a multiple of 64 tokens (one page per sub-tile), 2 smaller pages.
// INLOOP (with MASKED): the comparison variant that keeps the skip decision inside the loop: no list; the
// loop walks every causal block j <= i and tests j's mask bit (kept in LDS) at each step, skipping the
// compute and the loads of unselected blocks but not the step itself (its barrier and bookkeeping).
// Selected blocks see exactly the same arithmetic in the same order, so the outputs are identical.
template <int PAGE, bool MASKED, bool INLOOP, int HEADS>
__global__ __launch_bounds__(256 * HEADS, 2 / HEADS) void bsa_bf16_kernel(BsaArgs a) {
  constexpr int PARTS = 4 / HEADS;  // 1 KB load instructions per wave for each of K and V per sub-tile
  // Two buffers, each its own LDS object, so the loads into one are known not to alias reads of the other.
  __shared__ __align__(1024) uint8_t kbuf0[TILE], vbuf0[TILE], kbuf1[TILE], vbuf1[TILE];
  __shared__ uint16_t list[(MASKED && !INLOOP) ? kMaxList : 1];
  __shared__ uint32_t mbits[INLOOP ? HEADS * kMaxList / 32 : 1];
  __shared__ int list_len;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int hsel = HEADS == 2 ? wave >> 2 : 0;  // head of the workgroup this wave serves
  const int wq = HEADS == 2 ? wave & 3 : wave;   // 32-row slice of the query block
  const uint32_t mine = hsel ? kSelSecond : kSelFirst;

  // ---- work item (same order as the generic kernel: XCD-aware, KV-head-major, longest rows first);
  //      HEADS consecutive query heads of one KV group per workgroup
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
  // mask row of the workgroup's head t (rows of consecutive heads are NB * mask_words words apart)
  auto mask_row = [&](int t) { return a.mask + ((int64_t)(h0 + t) * a.NB + ib) * a.mask_words; };

  // ---- list of selected blocks (union over the workgroup's heads, one selection bit per head)
  int nsel;
  if constexpr (INLOOP) {
    if (wave == 0) {
      const int nwords = (i >> 5) + 1;
      for (int t = 0; t < HEADS; ++t)
        for (int w = lane; w < nwords; w += 64) mbits[t * (kMaxList / 32) + w] = mask_row(t)[w];
    }
    __syncthreads();
    nsel = i + 1;
  } else if constexpr (MASKED) {
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

  // ---- Q fragments (B operand of S^T = K Q^T)
  const int qr = wq * 32 + l32;
  const int qpos = i * B + qr;
  const bool qvalid = qpos < L;
  bf16x8 qf[8];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)(tb + qpos) * a.hq + h) * D;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      uint4 w = qvalid ? *(const uint4*)(qp + 16 * kk + 8 * half) : make_uint4(0u, 0u, 0u, 0u);
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- loader geometry: instruction m of this wave fills LDS chunk c = PARTS*wave + m = tile rows
  //      4c + lane/16, slot lane & 15 (16 bytes); the lane fetches the swizzled source chunk.
  //      Contiguous K/V and pages of >= 64 tokens: buffer loads whose base (the sub-tile's first row) is
  //      scalar and whose per-lane byte offsets never change, with the buffer size ending at the
  //      request's last row (rows past it read as zeros; they are causally masked).  Smaller pages: one
  //      page lookup per row and global addresses.
  const int64_t row_stride = (int64_t)a.hkv * D * 2;
  // (fixed size 4: lambdas that capture arrays of template-dependent size lose their host stubs)
  int ldrow[4], kchunk[4], vchunk[4], koff_ld[4], voff_ld[4];
#pragma unroll
  for (int m = 0; m < PARTS; ++m) {
    const int row = 4 * (PARTS * wave + m) + (lane >> 4);
    const int slot = lane & 15;
    ldrow[m] = row;
    kchunk[m] = slot ^ (row & 15);
    vchunk[m] = slot ^ (4 * (row & 3));
    koff_ld[m] = row * (int)row_stride + kchunk[m] * 16;
    voff_ld[m] = row * (int)row_stride + vchunk[m] * 16;
  }
  const uint8_t* kbase_all = (const uint8_t*)a.k;
  const uint8_t* vbase_all = (const uint8_t*)a.v;
  const int64_t head_off = (int64_t)g * D * 2;

  // list entry of sub-tile u: block index | selection bits
  auto entry = [&](int u) -> uint32_t {
    if constexpr (MASKED && !INLOOP) {
      return (uint32_t)list[u >> 1];
    } else if constexpr (INLOOP) {
      const int j = u >> 1;
      uint32_t e = (uint32_t)j;
      if ((mbits[j >> 5] >> (j & 31)) & 1u) e |= kSelFirst;
      if (HEADS == 2 && ((mbits[kMaxList / 32 + (j >> 5)] >> (j & 31)) & 1u)) e |= kSelSecond;
      return e;
    } else {
      return (uint32_t)(u >> 1) | kSelFirst | kSelSecond;
    }
  };
  // first key of sub-tile u; only list entries pack the block index (dense and in-loop steps walk j = u/2,
  // which may exceed the list's 14 bits)
  auto sub_key0 = [&](uint32_t e, int u) -> int {
    const int j = (MASKED && !INLOOP) ? (int)(e & kBlockBits) : (u >> 1);
    return j * B + (u & 1) * KT;
  };
  // must the workgroup load sub-tile u (in-loop variant: is its block selected by any head)?
  auto wanted = [&](uint32_t e) -> bool { return !INLOOP || (e & (kSelFirst | kSelSecond)) != 0; };

  // The loads of sub-tile u: part m fills LDS chunk m of this wave in K and in V.  kb/vb: the sub-tile's
  // first row (scalar); nrec: bytes up to the request's end.
  auto issue_part = [&](int kp0, int nrec, const uint8_t* kb, const uint8_t* vb, lds_u8* kl, lds_u8* vl, int m) {
    if (PAGE == 0 || PAGE == 1) {
      const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)kb, 0, nrec, kBufDword3);
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)vb, 0, nrec, kBufDword3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, kl + m * 1024, 16, koff_ld[m], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, vl + m * 1024, 16, voff_ld[m], 0, 0, 0);
    } else {
      const int kp = min(kp0 + ldrow[m], L - 1);
      const int page = a.kv.page_table[(int64_t)r * a.kv.pt_stride + kp / a.kv.page_size];
      const int64_t off = ((int64_t)page * a.kv.page_size + (kp % a.kv.page_size)) * row_stride + head_off;
      __builtin_amdgcn_global_load_lds((const void*)(kbase_all + off + kchunk[m] * 16), kl + m * 1024, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vbase_all + off + vchunk[m] * 16), vl + m * 1024, 16, 0, 0);
    }
  };
  // Scalar base of sub-tile u (contiguous K/V or one page of >= 64 tokens).
  auto tile_base = [&](int kp0) -> int64_t {
    int64_t tok0;  // token index (pool row) of the sub-tile's first key
    if (PAGE == 0) {
      tok0 = (int64_t)tb + kp0;
    } else if (PAGE == 1) {
      const int page = a.kv.page_table[(int64_t)r * a.kv.pt_stride + kp0 / a.kv.page_size];
      tok0 = (int64_t)page * a.kv.page_size + (kp0 % a.kv.page_size);
    } else {
      tok0 = 0;
    }
    return tok0 * row_stride + head_off;
  };
  auto issue_loads = [&](int u, uint8_t* kdst, uint8_t* vdst) {
    const uint32_t e = entry(u);
    const int kp0 = sub_key0(e, u);
    // a second half-block past the end of the request, or (in-loop variant) a block nobody selected
    if (kp0 >= L || !wanted(e)) return;
    const int64_t base = tile_base(kp0);
    const int nrec = min(L - kp0, KT) * (int)row_stride;
#pragma unroll
    for (int m = 0; m < PARTS; ++m)
      issue_part(kp0, nrec, kbase_all + base, vbase_all + base, (lds_u8*)kdst + wave * (PARTS * 1024),
                 (lds_u8*)vdst + wave * (PARTS * 1024), m);
  };

  // ---- operand read offsets (bytes inside a tile)
  // K (A operand of S^T): row 32t + l32, chunk c = 2kk + half at slot c ^ (row & 15); row & 15 = l32 & 15.
  uint32_t koffs[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) koffs[kk] = l32 * 256 + 16 * ((2 * kk + half) ^ (l32 & 15));
  // V^T (A operand of O^T) via transposing reads: source lane (G = lane/16, s = lane%16, rr = s/4, c = s%4)
  // addresses row 16mm + 4*(G/2) + rr (+8 for the second read), dims 32dt + 16*(G&1) + 4c.
  uint32_t voffs[4];
  {
    const int G = lane >> 4, s = lane & 15, rr = s >> 2, c = s & 3;
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
  float m_run = -1e30f;  // reference max (log2 units); finite so masked rows never form inf - inf
  float l_part = 0.f;
  const float c2 = a.scale_log2;

  // The compute of sub-tile u (K and V in kcur, vcur).
  auto compute = [&](int u, const uint8_t* kcur, const uint8_t* vcur) __attribute__((always_inline)) {
    const uint32_t e = entry(u);
    const int kp0 = sub_key0(e, u);
    const bool diag = (kp0 / B) == i;
    // nothing to compute: the sub-tile starts past the request's end, or (diagonal block) every key is
    // after the wave's rows, or the wave's head did not select the block
    const bool idle = kp0 >= L || (diag && kp0 > i * B + wq * 32 + 31) || !(e & mine);
    if (idle) return;
    const lds_u8* Kt = (const lds_u8*)kcur;
    const lds_u8* Vt = (const lds_u8*)vcur;
    f32x16 s0, s1;
    auto scores = [&]() {
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        s0[x] = 0.f;
        s1[x] = 0.f;
      }
      // K fragments are read two k-steps ahead of the MFMAs that use them (hides the LDS latency)
      bf16x8 ka[3], kb[3];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        ka[kk] = *(const __attribute__((address_space(3))) bf16x8*)(Kt + koffs[kk]);
        kb[kk] = *(const __attribute__((address_space(3))) bf16x8*)(Kt + koffs[kk] + 32 * 256);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        if (kk + 2 < 8) {
          ka[(kk + 2) % 3] = *(const __attribute__((address_space(3))) bf16x8*)(Kt + koffs[kk + 2]);
          kb[(kk + 2) % 3] = *(const __attribute__((address_space(3))) bf16x8*)(Kt + koffs[kk + 2] + 32 * 256);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk % 3], qf[kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[kk % 3], qf[kk], s1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
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
    // Move the reference max to this tile's max (the O^T, sum rescale by 2^(old - new) is exact).
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
    uint4 pw[4];  // P rounded to bf16 pairs, the B operand of each k-step
    // P = 2^(s c2 - m_run), packed; returns the sum of the rounded values (v_dot2_f32_bf16 with (1, 1)).
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
  };

  // One sub-tile: wait for its loads, start the next sub-tile's loads into the other buffer (free since
  // the barrier), compute.  With two heads and a list of at most 3/4 of the row's causal blocks, the
  // second head's waves issue their share of the next loads right after the barrier and the first head's
  // waves theirs at the end of the step: the second head's waves, which each SIMD's matrix pipe serves
  // last, then no longer queue behind the first head's loads in the memory pipe (about 2% faster at 25%
  // and 50% of the blocks; fuller rows, dense causal and the in-loop variant were slower that way and
  // issue all loads after the barrier).
  const bool at_end = HEADS == 2 && MASKED && !INLOOP && hsel == 0 && 4 * nsel <= 3 * (i + 1);
  auto step = [&](int u, const uint8_t* kcur, const uint8_t* vcur, uint8_t* knext, uint8_t* vnext) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (!at_end && u + 1 < nsub) issue_loads(u + 1, knext, vnext);
    compute(u, kcur, vcur);
    if (at_end && u + 1 < nsub) issue_loads(u + 1, knext, vnext);
  };

  if (nsub > 0) issue_loads(0, kbuf0, vbuf0);
  for (int u = 0; u < nsub; u += 2) {
    step(u, kbuf0, vbuf0, kbuf1, vbuf1);
    if (u + 1 < nsub) step(u + 1, kbuf1, vbuf1, kbuf0, vbuf0);
  }

  // ---- epilogue
  const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
  if (!qvalid) return;
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  const int64_t ooff = ((int64_t)(tb + qpos) * a.hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * dt + 8 * rq + 4 * half;
      *(uint2*)((uint16_t*)a.out + ooff + d0) =
          make_uint2(cvt_bf16x2(o[dt][4 * rq] * inv, o[dt][4 * rq + 1] * inv),
                     cvt_bf16x2(o[dt][4 * rq + 2] * inv, o[dt][4 * rq + 3] * inv));
    }
  if (a.lse != nullptr && half == 0)
    a.lse[(int64_t)h * a.tokens + tb + qpos] =
        (l_tot > 0.f) ? (m_run + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

bool bsa_bf16_supported(int dtype, int head_dim, int block) {
  return dtype == STEM_BF16 && head_dim == D && block == B;
}

template <bool MASKED, bool INLOOP, int HEADS>
static hipError_t launch_heads(const BsaArgs& args, hipStream_t s) {
  BsaArgs a = args;
  const int64_t wgs = (int64_t)(a.hq / HEADS) * a.NB;
  a.xcd_remap = wgs % 8 == 0 ? 1 : 0;
  const dim3 grid((unsigned)wgs), block(256 * HEADS);
  const int page_mode = !a.kv.paged ? 0 : (a.kv.page_size % KT == 0 ? 1 : 2);
  if (INLOOP || page_mode == 0) hipLaunchKernelGGL((bsa_bf16_kernel<0, MASKED, INLOOP, HEADS>), grid, block, 0, s, a);
  else if constexpr (!INLOOP) {  // the in-loop comparator takes contiguous K/V only
    if (page_mode == 1) hipLaunchKernelGGL((bsa_bf16_kernel<1, MASKED, INLOOP, HEADS>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((bsa_bf16_kernel<2, MASKED, INLOOP, HEADS>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// Two heads per workgroup whenever a KV group has an even number of query heads.
hipError_t launch_bsa_bf16(const BsaArgs& a, bool masked, hipStream_t s) {
  const bool pair = (a.hq / a.hkv) % 2 == 0;
  if (masked) return pair ? launch_heads<true, false, 2>(a, s) : launch_heads<true, false, 1>(a, s);
  return pair ? launch_heads<false, false, 2>(a, s) : launch_heads<false, false, 1>(a, s);
}

hipError_t launch_bsa_bf16_inloop(const BsaArgs& a, hipStream_t s) {
  return (a.hq / a.hkv) % 2 == 0 ? launch_heads<true, true, 2>(a, s) : launch_heads<true, true, 1>(a, s);
}

}  // namespace stem
