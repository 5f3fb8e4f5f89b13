/*
 * The C ABI used from plain C with the HIP runtime only (no Python, no PyTorch): mask,
 * forward with residual and backward on a small seeded problem, plus the documented error
 * returns.  Writes inputs and outputs to the file named on the command line so that a test
 * can run the same inputs through the Python binding and compare the results bit for bit.
 *
 * File layout (little endian): int32 B, H, N, d, blk_q, blk_k; then q, k, v, dout as bf16
 * bits [B,H,N,d]; kv_cnt int32 [B,H,Nqb]; kv_idx int32 [B,H,Nqb,Nkb]; o, o_lo bf16 bits;
 * lse fp32 [B,H,N]; dq, dk, dv fp32 [B,H,N,d].
 *
 * Exit status 0 when every call behaved as documented.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "spa.h"

#define CHECK_HIP(x)                                                               \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      exit(2);                                                                     \
    }                                                                              \
  } while (0)

#define EXPECT(cond, msg)                      \
  do {                                         \
    if (!(cond)) {                             \
      fprintf(stderr, "failed: %s\n", msg);    \
      exit(1);                                 \
    }                                          \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static double next_uniform(void) { /* xorshift64*, uniform in [0, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) * 0x1.0p-53;
}

static uint16_t to_bf16(float x) { /* round to nearest even (finite inputs) */
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static void* dev_copy(const void* host, size_t bytes) {
  void* p = NULL;
  CHECK_HIP(hipMalloc(&p, bytes));
  CHECK_HIP(hipMemcpy(p, host, bytes, hipMemcpyHostToDevice));
  return p;
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  CHECK_HIP(hipMalloc(&p, bytes));
  return p;
}

static void fetch(void* host, const void* dev, size_t bytes) {
  CHECK_HIP(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost));
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s OUTPUT_FILE\n", argv[0]);
    return 2;
  }
  spa_dims dm = {1, 2, 1000, 64, 64, 64}; /* ragged: 1000 = 15 * 64 + 40 */
  const int nqb = (dm.N + dm.blk_q - 1) / dm.blk_q, nkb = (dm.N + dm.blk_k - 1) / dm.blk_k;
  const size_t nel = (size_t)dm.B * dm.H * dm.N * dm.d;
  const size_t nrow = (size_t)dm.B * dm.H * dm.N;
  const size_t nlist = (size_t)dm.B * dm.H * nqb;

  /* inputs: uniform in [-1, 1); every query and the keys of key blocks 3 and 9 also get
     a shared component along (1, ..., 1), so that the pooled map is peaked and the lists
     are short */
  uint16_t* host_in[4];
  for (int t = 0; t < 4; ++t) {
    host_in[t] = (uint16_t*)malloc(nel * 2);
    for (size_t e = 0; e < nel; ++e) {
      double x = 2.0 * next_uniform() - 1.0;
      const int row = (int)((e / dm.d) % dm.N);
      if (t == 0) x += 0.5;
      if (t == 1 && (row / dm.blk_k == 3 || row / dm.blk_k == 9)) x += 1.5;
      host_in[t][e] = to_bf16((float)x);
    }
  }
  void* q = dev_copy(host_in[0], nel * 2);
  void* k = dev_copy(host_in[1], nel * 2);
  void* v = dev_copy(host_in[2], nel * 2);
  void* dout = dev_copy(host_in[3], nel * 2);

  /* documented error returns, before any work */
  spa_dims bad = dm;
  bad.d = 96;
  EXPECT(spa_mask_workspace_bytes(&bad) == 0, "workspace size of unsupported dims is 0");
  EXPECT(spa_bwd_workspace_bytes(&bad) == 0, "bwd workspace size of unsupported dims is 0");
  EXPECT(spa_status_string(SPA_E_NULL) != NULL, "status text");
  EXPECT(spa_version() > 0, "version");

  int32_t* kv_idx = (int32_t*)dev_alloc(nlist * nkb * 4);
  int32_t* kv_cnt = (int32_t*)dev_alloc(nlist * 4);
  const size_t mws_bytes = spa_mask_workspace_bytes(&dm);
  EXPECT(mws_bytes > 0, "mask workspace size");
  void* mws = dev_alloc(mws_bytes);
  EXPECT(spa_build_mask(&dm, NULL, k, 0.1, 0.9, 0.0, kv_idx, kv_cnt, NULL, mws, mws_bytes,
                        NULL) == SPA_E_NULL, "NULL q is rejected");
  EXPECT(spa_build_mask(&bad, q, k, 0.1, 0.9, 0.0, kv_idx, kv_cnt, NULL, mws, mws_bytes,
                        NULL) == SPA_E_UNSUPPORTED, "d = 96 is rejected");
  EXPECT(spa_build_mask(&dm, q, k, 1.5, 0.9, 0.0, kv_idx, kv_cnt, NULL, mws, mws_bytes,
                        NULL) == SPA_E_PARAM, "k_frac > 1 is rejected");
  EXPECT(spa_build_mask(&dm, q, k, 0.1, 0.9, 0.0, kv_idx, kv_cnt, NULL, mws, mws_bytes - 1,
                        NULL) == SPA_E_WORKSPACE, "short workspace is rejected");

  /* the hot path on the default stream */
  EXPECT(spa_build_mask(&dm, q, k, 0.1, 0.9, 0.0, kv_idx, kv_cnt, NULL, mws, mws_bytes,
                        NULL) == SPA_OK, "build_mask");
  void* o = dev_alloc(nel * 2);
  void* o_lo = dev_alloc(nel * 2);
  float* lse = (float*)dev_alloc(nrow * 4);
  const size_t fws_bytes = spa_fwd_workspace_bytes(&dm);
  EXPECT(fws_bytes > 0, "fwd workspace size");
  void* fws = dev_alloc(fws_bytes);
  EXPECT(spa_sparse_attn_fwd(&dm, q, k, v, kv_idx, kv_cnt, 0.0, o, o_lo, lse, NULL, 0, NULL) ==
             SPA_E_NULL, "the residual output needs the workspace");
  EXPECT(spa_sparse_attn_fwd(&dm, q, k, v, kv_idx, kv_cnt, 0.0, o, o_lo, lse, fws, fws_bytes - 1,
                             NULL) == SPA_E_WORKSPACE, "short forward workspace is rejected");
  EXPECT(spa_sparse_attn_fwd(&dm, q, k, v, kv_idx, kv_cnt, 0.0, o, o_lo, lse, fws, fws_bytes,
                             NULL) == SPA_OK, "sparse_attn_fwd");
  const size_t bws_bytes = spa_bwd_workspace_bytes(&dm);
  EXPECT(bws_bytes > 0, "bwd workspace size");
  void* bws = dev_alloc(bws_bytes);
  float* dq = (float*)dev_alloc(nel * 4);
  float* dk = (float*)dev_alloc(nel * 4);
  float* dv = (float*)dev_alloc(nel * 4);
  EXPECT(spa_sparse_attn_bwd(&dm, q, k, v, o, o_lo, dout, lse, kv_idx, kv_cnt, 0.0, dq, dk, dv,
                             0, bws, bws_bytes, NULL) == SPA_OK, "sparse_attn_bwd");
  CHECK_HIP(hipDeviceSynchronize());

  /* the staged calls, one stage per call into fresh outputs and workspaces, equal the
     unstaged calls byte for byte; bad stage masks are rejected before any launch */
  EXPECT(spa_sparse_attn_fwd_stages(&dm, q, k, v, kv_idx, kv_cnt, 0.0, o, o_lo, lse, fws,
                                    fws_bytes, 0u, NULL) == SPA_E_PARAM, "empty fwd stage mask");
  EXPECT(spa_sparse_attn_fwd_stages(&dm, q, k, v, kv_idx, kv_cnt, 0.0, o, o_lo, lse, fws,
                                    fws_bytes, 4u, NULL) == SPA_E_PARAM, "unknown fwd stage bit");
  EXPECT(spa_sparse_attn_bwd_stages(&dm, q, k, v, o, o_lo, dout, lse, kv_idx, kv_cnt, 0.0, dq,
                                    dk, dv, 0, bws, bws_bytes, 8u, NULL) == SPA_E_PARAM,
         "unknown bwd stage bit");
  void* o2 = dev_alloc(nel * 2);
  void* o_lo2 = dev_alloc(nel * 2);
  float* lse2 = (float*)dev_alloc(nrow * 4);
  void* fws2 = dev_alloc(fws_bytes);
  const unsigned fwd_st[2] = {SPA_FWD_PREP, SPA_FWD_ATTN};
  for (int t = 0; t < 2; ++t)
    EXPECT(spa_sparse_attn_fwd_stages(&dm, q, k, v, kv_idx, kv_cnt, 0.0, o2, o_lo2, lse2, fws2,
                                      fws_bytes, fwd_st[t], NULL) == SPA_OK,
           "staged sparse_attn_fwd");
  void* bws2 = dev_alloc(bws_bytes);
  float* dq2 = (float*)dev_alloc(nel * 4);
  float* dk2 = (float*)dev_alloc(nel * 4);
  float* dv2 = (float*)dev_alloc(nel * 4);
  const unsigned bwd_st[3] = {SPA_BWD_PREP, SPA_BWD_DQ, SPA_BWD_DKDV};
  for (int t = 0; t < 3; ++t)
    EXPECT(spa_sparse_attn_bwd_stages(&dm, q, k, v, o2, o_lo2, dout, lse2, kv_idx, kv_cnt, 0.0,
                                      dq2, dk2, dv2, 0, bws2, bws_bytes, bwd_st[t], NULL) ==
               SPA_OK,
           "staged sparse_attn_bwd");
  CHECK_HIP(hipDeviceSynchronize());
  {
    const void* pairs[][2] = {{o, o2}, {o_lo, o_lo2}, {lse, lse2}, {dq, dq2}, {dk, dk2},
                              {dv, dv2}};
    const size_t sizes[] = {nel * 2, nel * 2, nrow * 4, nel * 4, nel * 4, nel * 4};
    for (int t = 0; t < 6; ++t) {
      unsigned char* a = (unsigned char*)malloc(sizes[t]);
      unsigned char* b = (unsigned char*)malloc(sizes[t]);
      fetch(a, pairs[t][0], sizes[t]);
      fetch(b, pairs[t][1], sizes[t]);
      EXPECT(memcmp(a, b, sizes[t]) == 0, "staged calls equal the unstaged ones");
      free(a);
      free(b);
    }
  }
  void* staged_bufs[] = {o2, o_lo2, lse2, fws2, bws2, dq2, dk2, dv2};
  for (size_t i = 0; i < sizeof(staged_bufs) / sizeof(staged_bufs[0]); ++i)
    CHECK_HIP(hipFree(staged_bufs[i]));

  /* results: structural checks here, values compared by the calling test */
  int32_t* h_cnt = (int32_t*)malloc(nlist * 4);
  int32_t* h_idx = (int32_t*)malloc(nlist * nkb * 4);
  fetch(h_cnt, kv_cnt, nlist * 4);
  fetch(h_idx, kv_idx, nlist * nkb * 4);
  for (size_t r = 0; r < nlist; ++r) {
    EXPECT(h_cnt[r] >= 1 && h_cnt[r] <= nkb, "list length in [1, Nkb]");
    for (int e = 1; e < h_cnt[r]; ++e)
      EXPECT(h_idx[r * nkb + e] > h_idx[r * nkb + e - 1], "lists ascending");
  }
  uint16_t* h_o = (uint16_t*)malloc(nel * 2);
  uint16_t* h_olo = (uint16_t*)malloc(nel * 2);
  float* h_lse = (float*)malloc(nrow * 4);
  float* h_g[3];
  fetch(h_o, o, nel * 2);
  fetch(h_olo, o_lo, nel * 2);
  fetch(h_lse, lse, nrow * 4);
  const float* dgrads[3] = {dq, dk, dv};
  for (int t = 0; t < 3; ++t) {
    h_g[t] = (float*)malloc(nel * 4);
    fetch(h_g[t], dgrads[t], nel * 4);
    for (size_t e = 0; e < nel; ++e) EXPECT(isfinite(h_g[t][e]), "finite gradients");
  }
  for (size_t r = 0; r < nrow; ++r) EXPECT(isfinite(h_lse[r]), "finite LSE");

  FILE* f = fopen(argv[1], "wb");
  EXPECT(f != NULL, "open output file");
  const int32_t hdr[6] = {dm.B, dm.H, dm.N, dm.d, dm.blk_q, dm.blk_k};
  fwrite(hdr, 4, 6, f);
  for (int t = 0; t < 4; ++t) fwrite(host_in[t], 2, nel, f);
  fwrite(h_cnt, 4, nlist, f);
  fwrite(h_idx, 4, nlist * nkb, f);
  fwrite(h_o, 2, nel, f);
  fwrite(h_olo, 2, nel, f);
  fwrite(h_lse, 4, nrow, f);
  for (int t = 0; t < 3; ++t) fwrite(h_g[t], 4, nel, f);
  fclose(f);

  void* dev_bufs[] = {q, k, v, dout, kv_idx, kv_cnt, mws, o, o_lo, lse, fws, bws, dq, dk, dv};
  for (size_t i = 0; i < sizeof(dev_bufs) / sizeof(dev_bufs[0]); ++i)
    CHECK_HIP(hipFree(dev_bufs[i]));
  printf("abi_smoke ok: %d x %d lists, version %d\n", (int)nlist, nkb, spa_version());
  return 0;
}
