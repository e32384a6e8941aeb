/* A plain C99 client of libkvarn: the header compiles as C, the library links and its host-side
 * validation answers as documented (no GPU needed). With "run <in> <out>" it also drives one
 * prefill quantisation and one decode step on the GPU through nothing but the C ABI and the HIP
 * runtime's C API, reading its inputs from <in> and writing the fp32 outputs to <out>.
 *
 * <in>: int32 header {magic 0x4B56524E, v_bits, n_tiles, hkv, hq, batch, max_blocks,
 * num_blocks, head_dim D}, then fp16 k[n_tiles*128][hkv][D], fp16 v (same), int32
 * dst_blocks[n_tiles], int32 block_table[batch][max_blocks], int32 seq_lens[batch], fp16
 * q[batch][hq][D], fp16 staging_k[batch][hkv][128][D], fp16 staging_v (same), float sm_scale. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvarn.h"

#define CHECK(cond, code)                                                   \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);   \
      return code;                                                          \
    }                                                                       \
  } while (0)

static int host_checks(void) {
  kvarn_config cfg;
  kvarn_default_config(&cfg, 8);
  CHECK(kvarn_abi_version() == KVARN_ABI_VERSION, 10);
  CHECK(cfg.head_dim == KVARN_HEAD_DIM && cfg.block_tokens == KVARN_TILE_TOKENS, 11);
  CHECK(cfg.k_bits == 4 && cfg.v_bits == 2 && cfg.sinkhorn_iters == 4, 12);
  CHECK(kvarn_tile_bytes(&cfg) == KVARN_TILE_BYTES, 13);
  CHECK(kvarn_block_bytes(&cfg) == 8u * KVARN_TILE_BYTES, 14);
  cfg.v_bits = 4;
  CHECK(kvarn_tile_bytes(&cfg) == KVARN_TILE_BYTES_V4, 15);
  cfg.v_bits = 3;
  CHECK(kvarn_tile_bytes(&cfg) == 0, 16);
  kvarn_default_config(&cfg, 8);
  /* validation fails before anything is enqueued: no device memory is touched */
  void* fake = (void*)(uintptr_t)0x1000;
  CHECK(kvarn_quantize_tiles(NULL, fake, fake, 1024, 1, fake, fake, 1, NULL) ==
            KVARN_ERR_NULL_ARG, 17);
  CHECK(kvarn_quantize_tiles(&cfg, fake, NULL, 1024, 1, fake, fake, 1, NULL) ==
            KVARN_ERR_NULL_ARG, 18);
  CHECK(kvarn_quantize_tiles(&cfg, fake, fake, 512, 1, fake, fake, 1, NULL) ==
            KVARN_ERR_BAD_SHAPE, 19);
  CHECK(kvarn_quantize_tiles(&cfg, fake, fake, 1024, 0, NULL, NULL, 0, NULL) == KVARN_OK, 20);
  size_t ws = 0;
  CHECK(kvarn_decode_workspace_bytes(&cfg, 4, 32, 8, &ws) == KVARN_OK && ws > 0, 21);
  CHECK(kvarn_decode_workspace_bytes(&cfg, 4, 30, 8, &ws) == KVARN_ERR_BAD_SHAPE, 22);
  CHECK(kvarn_decode_attention(&cfg, fake, 32, fake, 1, fake, 8, fake, fake, fake, 0.1f,
                               (float*)fake, fake, 0, 4, NULL) == KVARN_ERR_WORKSPACE, 23);
  CHECK(strlen(kvarn_status_string(KVARN_ERR_UNSUPPORTED)) > 0, 24);
  /* every entry point's validation, including misaligned block pools */
  void* odd = (void*)(uintptr_t)0x1004;
  CHECK(kvarn_quantize_tiles(&cfg, fake, fake, 1024, 1, fake, odd, 1, NULL) ==
            KVARN_ERR_BAD_SHAPE, 25);
  CHECK(kvarn_append_token(&cfg, fake, fake, fake, fake, 4, fake, fake, odd, 8, 2, NULL) ==
            KVARN_ERR_BAD_SHAPE, 26);
  CHECK(kvarn_append_token(&cfg, fake, fake, fake, fake, 0, fake, fake, fake, 8, 2, NULL) ==
            KVARN_ERR_BAD_SHAPE, 27);
  CHECK(kvarn_decode_workspace_bytes(&cfg, 4, 32, 8, &ws) == KVARN_OK, 28);
  CHECK(kvarn_decode_attention(&cfg, fake, 32, odd, 1, fake, 8, fake, fake, fake, 0.1f,
                               (float*)fake, (void*)(uintptr_t)0x10000, ws, 4, NULL) ==
            KVARN_ERR_BAD_SHAPE, 29);
  size_t wsm = 0;
  CHECK(kvarn_decode_multi_workspace_bytes(&cfg, 4, 32, 4, 8, &wsm) == KVARN_OK && wsm > ws, 30);
  CHECK(kvarn_decode_multi_workspace_bytes(&cfg, 4, 32, KVARN_MAX_QUERY_TOKENS + 1, 8, &wsm) ==
            KVARN_ERR_BAD_SHAPE, 31);
  CHECK(kvarn_dequantize_tiles(&cfg, odd, 4, fake, 1, (float*)fake, (float*)fake, NULL) ==
            KVARN_ERR_BAD_SHAPE, 32);
  CHECK(kvarn_dequantize_tiles(&cfg, fake, 4, fake, 0, NULL, NULL, NULL) == KVARN_OK, 33);
  CHECK(kvarn_fp16_block_bytes(&cfg) == 8u * KVARN_FP16_RECORD_BYTES, 34);
  CHECK(kvarn_fp16_write_tiles(&cfg, fake, fake, 1024, 1, fake, odd, 1, NULL) ==
            KVARN_ERR_BAD_SHAPE, 35);
  CHECK(kvarn_decode_attention_fp16(&cfg, fake, 32, fake, 1, fake, 8, fake, fake, fake, 0.1f,
                                    (float*)fake, fake, 0, 4, NULL) == KVARN_ERR_WORKSPACE, 36);
  for (int st = 0; st <= 6; ++st) CHECK(kvarn_status_string((kvarn_status)st) != NULL, 37);
  /* head dimensions: record sizes 64 D + 16 D v_bits + 2 (D + 384), token stride >= hkv * D,
   * sign words past D / 32 rejected, the fp16 cache at 128 only */
  kvarn_default_config(&cfg, 8);
  cfg.head_dim = 64;
  CHECK(kvarn_tile_bytes(&cfg) == 7040u, 51);
  cfg.v_bits = 4;
  CHECK(kvarn_tile_bytes(&cfg) == 9088u, 52);
  cfg.head_dim = 256;
  CHECK(kvarn_tile_bytes(&cfg) == 34048u, 53);
  cfg.v_bits = 2;
  CHECK(kvarn_tile_bytes(&cfg) == 25856u, 54);
  CHECK(kvarn_quantize_tiles(&cfg, fake, fake, 8 * 128, 1, fake, fake, 1, NULL) ==
            KVARN_ERR_BAD_SHAPE, 55);
  cfg.rotation_signs[7] = 1u;
  CHECK(kvarn_tile_bytes(&cfg) > 0, 56);
  cfg.head_dim = 64;
  CHECK(kvarn_tile_bytes(&cfg) == 0, 57);
  cfg.rotation_signs[7] = 0u;
  CHECK(kvarn_fp16_block_bytes(&cfg) == 0, 58);
  CHECK(kvarn_decode_attention_fp16(&cfg, fake, 32, fake, 1, fake, 8, fake, fake, fake, 0.1f,
                                    (float*)fake, fake, 0, 4, NULL) == KVARN_ERR_UNSUPPORTED, 59);
  cfg.head_dim = 96;
  CHECK(kvarn_tile_bytes(&cfg) == 0 && kvarn_decode_workspace_bytes(&cfg, 4, 32, 8, &ws) ==
            KVARN_ERR_UNSUPPORTED, 60);
  return 0;
}

#ifdef KVARN_C_CLIENT_GPU
#include <hip/hip_runtime_api.h>

static void* upload(const void* host, size_t n) {
  void* d = NULL;
  if (hipMalloc(&d, n ? n : 16) != hipSuccess) return NULL;
  if (n && hipMemcpy(d, host, n, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

static int gpu_run(const char* in_path, const char* out_path) {
  FILE* f = fopen(in_path, "rb");
  CHECK(f != NULL, 30);
  int32_t h[9];
  CHECK(fread(h, sizeof h, 1, f) == 1 && h[0] == 0x4B56524E, 31);
  const int v_bits = h[1], n_tiles = h[2], hkv = h[3], hq = h[4], batch = h[5];
  const int max_blocks = h[6], num_blocks = h[7], d = h[8];
  CHECK(n_tiles >= 0 && hkv > 0 && hq > 0 && batch > 0 && max_blocks > 0 && num_blocks > 0 &&
            (d == 64 || d == 128 || d == 256), 32);
  const size_t kv_n = (size_t)n_tiles * 128 * hkv * d * 2;
  const size_t bt_n = (size_t)batch * max_blocks * 4;
  const size_t q_n = (size_t)batch * hq * d * 2;
  const size_t st_n = (size_t)batch * hkv * 128 * d * 2;
  char* buf = (char*)malloc(2 * kv_n + n_tiles * 4 + bt_n + batch * 4 + q_n + 2 * st_n + 4);
  CHECK(buf != NULL, 33);
  char* p = buf;
  const size_t total = 2 * kv_n + n_tiles * 4 + bt_n + batch * 4 + q_n + 2 * st_n + 4;
  CHECK(fread(buf, 1, total, f) == total, 34);
  fclose(f);
  kvarn_config cfg;
  kvarn_default_config(&cfg, hkv);
  cfg.v_bits = v_bits;
  cfg.head_dim = d;
  const size_t pool_n = (size_t)num_blocks * kvarn_block_bytes(&cfg);
  CHECK(pool_n > 0, 35);
  void* k = upload(p, kv_n); p += kv_n;
  void* v = upload(p, kv_n); p += kv_n;
  void* dst = upload(p, n_tiles * 4); p += n_tiles * 4;
  void* bt = upload(p, bt_n); p += bt_n;
  void* lens = upload(p, batch * 4); p += batch * 4;
  void* q = upload(p, q_n); p += q_n;
  void* sk = upload(p, st_n); p += st_n;
  void* sv = upload(p, st_n); p += st_n;
  float sm;
  memcpy(&sm, p, 4);
  void* pool = NULL;
  void* out = NULL;
  void* work = NULL;
  size_t ws = 0;
  CHECK(k && v && dst && bt && lens && q && sk && sv, 36);
  CHECK(hipMalloc(&pool, pool_n) == hipSuccess && hipMemset(pool, 0, pool_n) == hipSuccess, 37);
  CHECK(kvarn_decode_workspace_bytes(&cfg, batch, hq, max_blocks, &ws) == KVARN_OK, 38);
  CHECK(hipMalloc(&work, ws) == hipSuccess, 39);
  CHECK(hipMalloc(&out, (size_t)batch * hq * d * 4) == hipSuccess, 40);
  CHECK(kvarn_quantize_tiles(&cfg, k, v, (int64_t)hkv * d, n_tiles, (const int32_t*)dst, pool,
                             num_blocks, NULL) == KVARN_OK, 41);
  CHECK(kvarn_decode_attention(&cfg, q, hq, pool, num_blocks, (const int32_t*)bt, max_blocks,
                               (const int32_t*)lens, sk, sv, sm, (float*)out, work, ws, batch,
                               NULL) == KVARN_OK, 42);
  CHECK(hipDeviceSynchronize() == hipSuccess, 43);
  float* host_out = (float*)malloc((size_t)batch * hq * d * 4);
  CHECK(host_out != NULL, 44);
  CHECK(hipMemcpy(host_out, out, (size_t)batch * hq * d * 4, hipMemcpyDeviceToHost) ==
            hipSuccess, 45);
  unsigned char* host_pool = (unsigned char*)malloc(pool_n);
  CHECK(host_pool != NULL, 46);
  CHECK(hipMemcpy(host_pool, pool, pool_n, hipMemcpyDeviceToHost) == hipSuccess, 47);
  FILE* o = fopen(out_path, "wb");
  CHECK(o != NULL, 48);
  CHECK(fwrite(host_out, 4, (size_t)batch * hq * d, o) == (size_t)batch * hq * d, 49);
  CHECK(fwrite(host_pool, 1, pool_n, o) == pool_n, 50);
  fclose(o);
  hipFree(k); hipFree(v); hipFree(dst); hipFree(bt); hipFree(lens); hipFree(q); hipFree(sk);
  hipFree(sv); hipFree(pool); hipFree(out); hipFree(work);
  free(buf); free(host_out); free(host_pool);
  return 0;
}
#endif

int main(int argc, char** argv) {
  int rc = host_checks();
  if (rc != 0) return rc;
  if (argc == 4 && strcmp(argv[1], "run") == 0) {
#ifdef KVARN_C_CLIENT_GPU
    rc = gpu_run(argv[2], argv[3]);
    if (rc != 0) return rc;
#else
    fprintf(stderr, "built without the HIP runtime\n");
    return 2;
#endif
  }
  printf("kvarn C client ok\n");
  return 0;
}
