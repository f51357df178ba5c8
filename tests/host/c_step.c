/*
 * One LCSA streaming step driven from plain C11 through include/lcsa.h and
 * the HIP runtime's C API, with no Python or torch: device buffers from
 * hipMalloc, the ring cache primed with 2 temporal blocks (4 latent frames),
 * then the chunk's 2 frames: partition + pool, draft top-k, attention with q
 * read in token layout, all on the null stream.
 *
 * Geometry: 1 batch, 2 heads, head_dim 64, bf16, 32 x 48 tokens (4 x 6
 * blocks), window 5, k = 1/3 of each row's candidates. Inputs are uniform in
 * [-1, 1) from xorshift32 (seed 2024), rounded to bf16 to nearest even.
 *
 * argv[1]: output file. It receives, in order: int32 header {T, H, W, NH, D,
 * kmax}; q, k, v for the 6 frames (uint16 bf16 bits, token layout); sel_cnt
 * (int32 [NH][nq]); sel_idx (int32 [NH][nq][kmax]); out (uint16, the chunk's
 * 2 frames); lse (float32 [NH][nq][128]). Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lcsa.h"

#define CHECK_HIP(x)                                                          \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "HIP error %d at line %d: %s\n", (int)e_, __LINE__,     \
              hipGetErrorString(e_));                                         \
      return 1;                                                               \
    }                                                                         \
  } while (0)
#define CHECK_LCSA(x)                                                         \
  do {                                                                        \
    lcsa_status s_ = (x);                                                     \
    if (s_ != LCSA_OK) {                                                      \
      fprintf(stderr, "lcsa status %d at line %d: %s\n", (int)s_, __LINE__,   \
              lcsa_last_error());                                             \
      return 1;                                                               \
    }                                                                         \
  } while (0)

static uint32_t rng = 2024u;
static uint32_t xorshift32(void) {
  rng ^= rng << 13;
  rng ^= rng >> 17;
  rng ^= rng << 5;
  return rng;
}

/* float32 -> bf16 bits, round to nearest even (inputs are finite) */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static int write_all(FILE* f, const void* p, size_t bytes) {
  return fwrite(p, 1, bytes, f) == bytes ? 0 : 1;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: c_step OUTPUT\n");
    return 2;
  }
  enum { NH = 2, D = 64, H = 32, W = 48, T_CACHE = 4, T_CHUNK = 2, T = 6, N_SLOTS = 4 };
  const int32_t nby = H / 8, nbx = W / 8, nS = nby * nbx, nq = (T_CHUNK / 2) * nS;
  const size_t frame = (size_t)H * W * NH * D;  /* elements of one latent frame */
  const size_t n_in = frame * T;

  uint16_t* host[3];
  for (int t = 0; t < 3; ++t) {
    host[t] = (uint16_t*)malloc(n_in * sizeof(uint16_t));
    if (!host[t]) return 1;
    for (size_t i = 0; i < n_in; ++i)
      host[t][i] = to_bf16((float)((double)xorshift32() / 2147483648.0 - 1.0));
  }
  void* dev[3];
  for (int t = 0; t < 3; ++t) {
    CHECK_HIP(hipMalloc(&dev[t], n_in * sizeof(uint16_t)));
    CHECK_HIP(hipMemcpy(dev[t], host[t], n_in * sizeof(uint16_t), hipMemcpyHostToDevice));
  }

  /* the ring: N_SLOTS temporal blocks of K, V^T and the pooled K */
  const size_t blocks = (size_t)NH * N_SLOTS * nS;
  const size_t bytes_kv = blocks * 128 * D * 2, bytes_pool = blocks * D * sizeof(double);
  void *k_ring, *v_ring, *kpool;
  CHECK_HIP(hipMalloc(&k_ring, bytes_kv));
  CHECK_HIP(hipMalloc(&v_ring, bytes_kv));
  CHECK_HIP(hipMalloc(&kpool, bytes_pool));
  lcsa_kv_cache cache;
  CHECK_LCSA(lcsa_kv_cache_init(&cache, 1, NH, D, nby, nbx, LCSA_BF16, N_SLOTS, k_ring, v_ring,
                                (double*)kpool, bytes_kv, bytes_kv, bytes_pool));

  /* prime the cache with frames 0..3 (temporal blocks 0 and 1) */
  int32_t slot = 0;
  CHECK_LCSA(lcsa_kv_cache_append(&cache, T_CACHE / 2, 0, &slot));
  lcsa_geom gc = {1, NH, D, T_CACHE, H, W, LCSA_BF16};
  CHECK_LCSA(lcsa_partition_pool(&gc, NULL, dev[1], dev[2], NULL, NULL, &cache, slot, NULL));

  /* the chunk: frames 4..5, temporal block 2 */
  const size_t off = frame * T_CACHE * sizeof(uint16_t);
  const char* q = (const char*)dev[0] + off;
  const char* k = (const char*)dev[1] + off;
  const char* v = (const char*)dev[2] + off;
  CHECK_LCSA(lcsa_kv_cache_append(&cache, T_CHUNK / 2, T_CACHE / 2, &slot));
  lcsa_geom g = {1, NH, D, T_CHUNK, H, W, LCSA_BF16};
  double* q_pool;
  CHECK_HIP(hipMalloc((void**)&q_pool, (size_t)NH * nq * D * sizeof(double)));
  CHECK_LCSA(lcsa_partition_pool(&g, q, k, v, NULL, q_pool, &cache, slot, NULL));

  lcsa_select_params p = {5, LCSA_BORDER_PRESERVED, 0, 1, 3, 0, 768, 1280, 768, 1280, 0};
  int32_t kmax = 0;
  CHECK_LCSA(lcsa_max_topk(&g, T_CACHE / 2, &cache, &p, &kmax));
  int32_t *sel_idx, *sel_cnt;
  CHECK_HIP(hipMalloc((void**)&sel_idx, (size_t)NH * nq * kmax * sizeof(int32_t)));
  CHECK_HIP(hipMalloc((void**)&sel_cnt, (size_t)NH * nq * sizeof(int32_t)));
  CHECK_LCSA(lcsa_draft_mask(&g, q_pool, T_CACHE / 2, &cache, &p, kmax, sel_idx, sel_cnt, NULL, 0,
                             NULL, 0, NULL));

  void* out;
  float* lse;
  const size_t n_out = frame * T_CHUNK;
  CHECK_HIP(hipMalloc(&out, n_out * sizeof(uint16_t)));
  CHECK_HIP(hipMalloc((void**)&lse, (size_t)NH * nq * 128 * sizeof(float)));
  CHECK_LCSA(lcsa_block_sparse_attn_tok(&g, q, &cache, sel_idx, sel_cnt, kmax, 0.0f, out, lse,
                                        NULL));
  CHECK_HIP(hipDeviceSynchronize());

  int32_t* h_cnt = (int32_t*)malloc((size_t)NH * nq * sizeof(int32_t));
  int32_t* h_idx = (int32_t*)malloc((size_t)NH * nq * kmax * sizeof(int32_t));
  uint16_t* h_out = (uint16_t*)malloc(n_out * sizeof(uint16_t));
  float* h_lse = (float*)malloc((size_t)NH * nq * 128 * sizeof(float));
  if (!h_cnt || !h_idx || !h_out || !h_lse) return 1;
  CHECK_HIP(hipMemcpy(h_cnt, sel_cnt, (size_t)NH * nq * sizeof(int32_t), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(h_idx, sel_idx, (size_t)NH * nq * kmax * sizeof(int32_t),
                      hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(h_out, out, n_out * sizeof(uint16_t), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(h_lse, lse, (size_t)NH * nq * 128 * sizeof(float), hipMemcpyDeviceToHost));

  FILE* f = fopen(argv[1], "wb");
  if (!f) return 1;
  const int32_t header[6] = {T, H, W, NH, D, kmax};
  int bad = write_all(f, header, sizeof header);
  for (int t = 0; t < 3; ++t) bad |= write_all(f, host[t], n_in * sizeof(uint16_t));
  bad |= write_all(f, h_cnt, (size_t)NH * nq * sizeof(int32_t));
  bad |= write_all(f, h_idx, (size_t)NH * nq * kmax * sizeof(int32_t));
  bad |= write_all(f, h_out, n_out * sizeof(uint16_t));
  bad |= write_all(f, h_lse, (size_t)NH * nq * 128 * sizeof(float));
  bad |= fclose(f) != 0;
  if (bad) return 1;

  for (int t = 0; t < 3; ++t) {
    CHECK_HIP(hipFree(dev[t]));
    free(host[t]);
  }
  CHECK_HIP(hipFree(k_ring));
  CHECK_HIP(hipFree(v_ring));
  CHECK_HIP(hipFree(kpool));
  CHECK_HIP(hipFree(q_pool));
  CHECK_HIP(hipFree(sel_idx));
  CHECK_HIP(hipFree(sel_cnt));
  CHECK_HIP(hipFree(out));
  CHECK_HIP(hipFree(lse));
  free(h_cnt);
  free(h_idx);
  free(h_out);
  free(h_lse);
  printf("c step ok: kmax %d\n", kmax);
  return 0;
}
