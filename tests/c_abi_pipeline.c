/* A plain C99 program that runs the whole path through include/stem.h on the GPU: stem_score,
 * stem_tpd_topk and bsa_prefill on one request of bf16 Q/K/V, with device memory from the HIP runtime's
 * C API.  Usage:  c_abi_pipeline <dir> <len> <hq> <hkv>
 * Reads <dir>/q.bin, k.bin, v.bin (bf16 bits, layouts of stem.h, head_dim 128, block 128), writes
 * <dir>/mask.bin (uint32 [hq][n][words]), counts.bin (int32 [hq][n]), out.bin (bf16 bits [len][hq][128])
 * and lse.bin (float [hq][len]).  Budget 25%, mu 7/10, beta 0.2.  Exit status 0 on success. */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "stem.h"

#define D 128

static int fail(const char* what, int st) {
  fprintf(stderr, "%s failed: %d (%s) %s\n", what, st, stem_status_string(st), stem_last_error());
  return 1;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof(path), "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* buf = malloc(bytes);
  const size_t got = buf ? fread(buf, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(buf);
    return NULL;
  }
  return buf;
}

static int write_file(const char* dir, const char* name, const void* data, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof(path), "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  const size_t put = fwrite(data, 1, bytes, f);
  fclose(f);
  return put != bytes;
}

int main(int argc, char** argv) {
  if (argc != 5) {
    fprintf(stderr, "usage: %s <dir> <len> <hq> <hkv>\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  const int len = atoi(argv[2]), hq = atoi(argv[3]), hkv = atoi(argv[4]);
  const int32_t cu[2] = {0, len};
  stem_problem p = {0};
  p.num_reqs = 1;
  p.cu_seqlens = cu;
  p.hq = hq;
  p.hkv = hkv;
  p.head_dim = D;
  p.block = 128;
  p.dtype = STEM_BF16;

  int64_t nb = 0;
  int32_t n = 0;
  int st = stem_block_counts(&p, &nb, &n);
  if (st != STEM_OK) return fail("stem_block_counts", st);
  const int words = (n + 31) / 32;
  const size_t qb = (size_t)len * hq * D * 2, kvb = (size_t)len * hkv * D * 2;
  void *hq_in = read_file(dir, "q.bin", qb), *hk_in = read_file(dir, "k.bin", kvb),
       *hv_in = read_file(dir, "v.bin", kvb);
  if (!hq_in || !hk_in || !hv_in) {
    fprintf(stderr, "cannot read the inputs\n");
    return 1;
  }
  const size_t ws_bytes = stem_workspace_bytes(&p);
  void *q, *k, *v, *ws, *out;
  float *scores, *lse;
  uint32_t* mask;
  int32_t* counts;
  if (hipMalloc(&q, qb) != hipSuccess || hipMalloc(&k, kvb) != hipSuccess || hipMalloc(&v, kvb) != hipSuccess ||
      hipMalloc(&ws, ws_bytes) != hipSuccess || hipMalloc((void**)&scores, (size_t)hq * n * n * 4) != hipSuccess ||
      hipMalloc((void**)&mask, (size_t)hq * n * words * 4) != hipSuccess ||
      hipMalloc((void**)&counts, (size_t)hq * n * 4) != hipSuccess || hipMalloc(&out, qb) != hipSuccess ||
      hipMalloc((void**)&lse, (size_t)hq * len * 4) != hipSuccess) {
    fprintf(stderr, "hipMalloc failed\n");
    return 1;
  }
  if (hipMemcpy(q, hq_in, qb, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(k, hk_in, kvb, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(v, hv_in, kvb, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "hipMemcpy failed\n");
    return 1;
  }
  st = stem_score(&p, q, k, v, 0.2f, scores, n, ws, ws_bytes, NULL);
  if (st != STEM_OK) return fail("stem_score", st);
  st = stem_tpd_topk(&p, scores, n, 25, 100, 7, 10, mask, words, counts, NULL);
  if (st != STEM_OK) return fail("stem_tpd_topk", st);
  st = bsa_prefill(&p, q, k, v, mask, words, 0.f, out, lse, NULL);
  if (st != STEM_OK) return fail("bsa_prefill", st);
  if (hipDeviceSynchronize() != hipSuccess) {
    fprintf(stderr, "hipDeviceSynchronize failed\n");
    return 1;
  }
  const size_t mb = (size_t)hq * n * words * 4, cb = (size_t)hq * n * 4, lb = (size_t)hq * len * 4;
  void *hm = malloc(mb), *hc = malloc(cb), *ho = malloc(qb), *hl = malloc(lb);
  if (!hm || !hc || !ho || !hl || hipMemcpy(hm, mask, mb, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(hc, counts, cb, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(ho, out, qb, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(hl, lse, lb, hipMemcpyDeviceToHost) != hipSuccess) {
    fprintf(stderr, "copy back failed\n");
    return 1;
  }
  if (write_file(dir, "mask.bin", hm, mb) || write_file(dir, "counts.bin", hc, cb) ||
      write_file(dir, "out.bin", ho, qb) || write_file(dir, "lse.bin", hl, lb)) {
    fprintf(stderr, "cannot write the outputs\n");
    return 1;
  }
  hipFree(q);
  hipFree(k);
  hipFree(v);
  hipFree(ws);
  hipFree(scores);
  hipFree(mask);
  hipFree(counts);
  hipFree(out);
  hipFree(lse);
  printf("c pipeline ok: %d tokens, %d blocks, %d query heads\n", len, n, hq);
  return 0;
}
