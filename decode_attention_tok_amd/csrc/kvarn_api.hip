// libkvarn C ABI: argument validation and kernel launches (declared in include/kvarn.h).

#include "../../include/kvarn.h"
#include "kvarn_kernels.hpp"

#include <stdint.h>

#include <algorithm>
#include <mutex>

namespace {

// Decode scratch for callers that cannot allocate (kvarn_decode_attention_noalloc): one array
// of KVARN_STATIC_SCRATCH_BYTES on every device the library runs on, held until the process
// ends. In host code the array's name is only a stand-in; its device address comes from
// hipGetSymbolAddress, taken once per device with that device current and kept per device.
__device__ __align__(256) unsigned char scratch[KVARN_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

kvarn_status scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return KVARN_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return KVARN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return KVARN_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVARN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kvarn_status check_config(const kvarn_config* cfg) {
  if (cfg == nullptr) return KVARN_ERR_NULL_ARG;
  if (cfg->num_kv_heads < 1) return KVARN_ERR_BAD_SHAPE;
  if ((cfg->head_dim != 64 && cfg->head_dim != 128 && cfg->head_dim != 256) ||
      cfg->block_tokens != KVARN_TILE_TOKENS || cfg->k_bits != 4 ||
      (cfg->v_bits != 2 && cfg->v_bits != 4) || cfg->sinkhorn_iters < 1 ||
      cfg->sinkhorn_iters > 16)
    return KVARN_ERR_UNSUPPORTED;
  for (int i = cfg->head_dim / 32; i < KVARN_SIGN_WORDS; ++i)   // words past the channels
    if (cfg->rotation_signs[i] != 0) return KVARN_ERR_UNSUPPORTED;
  return KVARN_OK;
}

kvarn_status from_hip(hipError_t e) { return e == hipSuccess ? KVARN_OK : KVARN_ERR_HIP; }

// Record bytes of a checked config (head dimension D): 64 D key-code bytes, 16 D per value
// bit, two metadata halves of D + 384 bytes.
size_t record_bytes(const kvarn_config* cfg) {
  const size_t d = (size_t)cfg->head_dim;
  return 64u * d + 16u * d * (size_t)cfg->v_bits + 2u * (d + 384u);
}

constexpr long long kMaxGrid = 0x7FFFFFFFLL;

}  // namespace

extern "C" {

void kvarn_default_config(kvarn_config* cfg, int32_t num_kv_heads) {
  if (cfg == nullptr) return;
  cfg->num_kv_heads = num_kv_heads;
  cfg->head_dim = KVARN_HEAD_DIM;
  cfg->block_tokens = KVARN_TILE_TOKENS;
  cfg->k_bits = 4;
  cfg->v_bits = 2;
  cfg->sinkhorn_iters = 4;
  for (int i = 0; i < KVARN_SIGN_WORDS; ++i) cfg->rotation_signs[i] = 0;
}

size_t kvarn_tile_bytes(const kvarn_config* cfg) {
  return check_config(cfg) == KVARN_OK ? record_bytes(cfg) : 0;
}

size_t kvarn_block_bytes(const kvarn_config* cfg) {
  return check_config(cfg) == KVARN_OK ? record_bytes(cfg) * (size_t)cfg->num_kv_heads : 0;
}

kvarn_status kvarn_quantize_tiles(const kvarn_config* cfg, const void* k, const void* v,
                                  int64_t token_stride, int32_t n_tiles,
                                  const int32_t* dst_blocks, void* block_pool,
                                  int64_t num_blocks, void* stream) {
  kvarn_status st = check_config(cfg);
  if (st != KVARN_OK) return st;
  if (n_tiles < 0 || num_blocks < 0) return KVARN_ERR_BAD_SHAPE;
  if (n_tiles == 0) return KVARN_OK;
  if (k == nullptr || v == nullptr || dst_blocks == nullptr || block_pool == nullptr)
    return KVARN_ERR_NULL_ARG;
  if (token_stride < (int64_t)cfg->num_kv_heads * cfg->head_dim || token_stride % 8 != 0 ||
      !aligned16(k) || !aligned16(v) || !aligned16(block_pool))
    return KVARN_ERR_BAD_SHAPE;
  if (2LL * cfg->num_kv_heads * n_tiles > kMaxGrid) return KVARN_ERR_BAD_SHAPE;
  return from_hip(kvarn::launch_quantize_tiles(
      static_cast<const __half*>(k), static_cast<const __half*>(v), token_stride, n_tiles,
      cfg->num_kv_heads, dst_blocks, static_cast<uint8_t*>(block_pool), num_blocks,
      cfg->sinkhorn_iters, cfg->rotation_signs, cfg->v_bits, cfg->head_dim,
      static_cast<hipStream_t>(stream)));
}

kvarn_status kvarn_append_token(const kvarn_config* cfg, const void* k_new, const void* v_new,
                                const int32_t* positions, const int32_t* block_table,
                                int32_t max_blocks_per_seq, void* staging_k, void* staging_v,
                                void* block_pool, int64_t num_blocks, int32_t batch,
                                void* stream) {
  kvarn_status st = check_config(cfg);
  if (st != KVARN_OK) return st;
  if (batch < 0 || max_blocks_per_seq < 1 || num_blocks < 0) return KVARN_ERR_BAD_SHAPE;
  if (batch == 0) return KVARN_OK;
  if (k_new == nullptr || v_new == nullptr || positions == nullptr || block_table == nullptr ||
      staging_k == nullptr || staging_v == nullptr || block_pool == nullptr)
    return KVARN_ERR_NULL_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(staging_k) || !aligned16(staging_v) ||
      !aligned16(block_pool))
    return KVARN_ERR_BAD_SHAPE;
  if (2LL * cfg->num_kv_heads * batch > kMaxGrid) return KVARN_ERR_BAD_SHAPE;
  return from_hip(kvarn::launch_append_token(
      static_cast<const __half*>(k_new), static_cast<const __half*>(v_new), positions,
      block_table, max_blocks_per_seq, static_cast<__half*>(staging_k),
      static_cast<__half*>(staging_v), static_cast<uint8_t*>(block_pool), num_blocks,
      cfg->num_kv_heads, batch, cfg->sinkhorn_iters, cfg->rotation_signs, cfg->v_bits,
      cfg->head_dim, static_cast<hipStream_t>(stream)));
}

namespace {

kvarn_status multi_workspace_bytes(const kvarn_config* cfg, int32_t batch, int32_t num_q_heads,
                                   int32_t n_query, int32_t max_blocks_per_seq, size_t* bytes) {
  kvarn_status st = check_config(cfg);
  if (st != KVARN_OK) return st;
  if (bytes == nullptr) return KVARN_ERR_NULL_ARG;
  if (batch < 0 || max_blocks_per_seq < 1 || num_q_heads < cfg->num_kv_heads ||
      num_q_heads % cfg->num_kv_heads != 0 ||
      num_q_heads / cfg->num_kv_heads > kvarn::kMaxGroup || n_query < 1 ||
      n_query > kvarn::kMaxQuery)
    return KVARN_ERR_BAD_SHAPE;
  // the packed decode's partial slots per row; the fp16 comparison decode of the same sizes
  // runs the split grid: the size covers both, so one workspace serves either call
  const int splits = std::max(
      kvarn::decode_slots(batch, cfg->num_kv_heads, max_blocks_per_seq,
                          num_q_heads / cfg->num_kv_heads * n_query, cfg->v_bits, cfg->head_dim),
      kvarn::decode_splits(batch, cfg->num_kv_heads, max_blocks_per_seq));
  *bytes = (size_t)batch * (size_t)n_query * (size_t)num_q_heads * (size_t)splits *
           (size_t)kvarn::partial_floats(cfg->head_dim) * sizeof(float);
  return KVARN_OK;
}

kvarn_status decode_multi(const kvarn_config* cfg, const void* q, int32_t num_q_heads,
                          int32_t n_query, const void* block_pool, int64_t num_blocks,
                          const int32_t* block_table, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, const void* staging_k, const void* staging_v,
                          float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                          int32_t batch, void* stream) {
  size_t need = 0;
  kvarn_status st = multi_workspace_bytes(cfg, batch, num_q_heads, n_query, max_blocks_per_seq,
                                          &need);
  if (st != KVARN_OK) return st;
  if (num_blocks < 0) return KVARN_ERR_BAD_SHAPE;
  if (batch == 0) return KVARN_OK;
  if (q == nullptr || block_pool == nullptr || block_table == nullptr || seq_lens == nullptr ||
      staging_k == nullptr || staging_v == nullptr || out == nullptr)
    return KVARN_ERR_NULL_ARG;
  if (workspace == nullptr || workspace_bytes < need) return KVARN_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KVARN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(staging_k) || !aligned16(staging_v) || !aligned16(out) ||
      !aligned16(block_pool))
    return KVARN_ERR_BAD_SHAPE;
  if (!(sm_scale == sm_scale)) return KVARN_ERR_BAD_SHAPE;
  const int splits = kvarn::decode_slots(batch, cfg->num_kv_heads, max_blocks_per_seq,
                                         num_q_heads / cfg->num_kv_heads * n_query, cfg->v_bits,
                                         cfg->head_dim);
  if ((long long)batch > 65535 || cfg->num_kv_heads > 65535) return KVARN_ERR_BAD_SHAPE;
  return from_hip(kvarn::launch_decode(
      static_cast<const __half*>(q), num_q_heads, cfg->num_kv_heads, n_query,
      static_cast<const uint8_t*>(block_pool), num_blocks, block_table, max_blocks_per_seq,
      seq_lens, static_cast<const __half*>(staging_k), static_cast<const __half*>(staging_v),
      sm_scale, out, static_cast<float*>(workspace), splits, batch, cfg->rotation_signs,
      cfg->v_bits, cfg->head_dim, static_cast<hipStream_t>(stream)));
}

}  // namespace

kvarn_status kvarn_decode_workspace_bytes(const kvarn_config* cfg, int32_t batch,
                                          int32_t num_q_heads, int32_t max_blocks_per_seq,
                                          size_t* bytes) {
  return multi_workspace_bytes(cfg, batch, num_q_heads, 1, max_blocks_per_seq, bytes);
}

kvarn_status kvarn_decode_attention(const kvarn_config* cfg, const void* q, int32_t num_q_heads,
                                    const void* block_pool, int64_t num_blocks,
                                    const int32_t* block_table, int32_t max_blocks_per_seq,
                                    const int32_t* seq_lens, const void* staging_k,
                                    const void* staging_v, float sm_scale, float* out,
                                    void* workspace, size_t workspace_bytes, int32_t batch,
                                    void* stream) {
  return decode_multi(cfg, q, num_q_heads, 1, block_pool, num_blocks, block_table,
                      max_blocks_per_seq, seq_lens, staging_k, staging_v, sm_scale, out,
                      workspace, workspace_bytes, batch, stream);
}

kvarn_status kvarn_decode_attention_noalloc(const kvarn_config* cfg, const void* q,
                                            int32_t num_q_heads, const void* block_pool,
                                            int64_t num_blocks, const int32_t* block_table,
                                            int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                            const void* staging_k, const void* staging_v,
                                            float sm_scale, float* out, int32_t batch,
                                            void* stream) {
  size_t need = 0;
  kvarn_status st = multi_workspace_bytes(cfg, batch, num_q_heads, 1, max_blocks_per_seq, &need);
  if (st != KVARN_OK) return st;
  if (batch == 0) return KVARN_OK;
  if (need > (size_t)KVARN_STATIC_SCRATCH_BYTES) return KVARN_ERR_SCRATCH_LIMIT;
  // every other argument is checked by the shared path before anything is launched; the
  // scratch address is only resolved once they have passed
  if (q == nullptr || block_pool == nullptr || block_table == nullptr || seq_lens == nullptr ||
      staging_k == nullptr || staging_v == nullptr || out == nullptr)
    return KVARN_ERR_NULL_ARG;
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != KVARN_OK) return st;
  return decode_multi(cfg, q, num_q_heads, 1, block_pool, num_blocks, block_table,
                      max_blocks_per_seq, seq_lens, staging_k, staging_v, sm_scale, out, ws,
                      (size_t)KVARN_STATIC_SCRATCH_BYTES, batch, stream);
}

kvarn_status kvarn_decode_multi_workspace_bytes(const kvarn_config* cfg, int32_t batch,
                                                int32_t num_q_heads, int32_t n_query,
                                                int32_t max_blocks_per_seq, size_t* bytes) {
  return multi_workspace_bytes(cfg, batch, num_q_heads, n_query, max_blocks_per_seq, bytes);
}

kvarn_status kvarn_decode_attention_multi(const kvarn_config* cfg, const void* q,
                                          int32_t num_q_heads, int32_t n_query,
                                          const void* block_pool, int64_t num_blocks,
                                          const int32_t* block_table, int32_t max_blocks_per_seq,
                                          const int32_t* seq_lens, const void* staging_k,
                                          const void* staging_v, float sm_scale, float* out,
                                          void* workspace, size_t workspace_bytes, int32_t batch,
                                          void* stream) {
  return decode_multi(cfg, q, num_q_heads, n_query, block_pool, num_blocks, block_table,
                      max_blocks_per_seq, seq_lens, staging_k, staging_v, sm_scale, out,
                      workspace, workspace_bytes, batch, stream);
}

kvarn_status kvarn_dequantize_tiles(const kvarn_config* cfg, const void* block_pool,
                                    int64_t num_blocks, const int32_t* src_blocks,
                                    int32_t n_tiles, float* k_out, float* v_out, void* stream) {
  kvarn_status st = check_config(cfg);
  if (st != KVARN_OK) return st;
  if (n_tiles < 0 || num_blocks < 0) return KVARN_ERR_BAD_SHAPE;
  if (n_tiles == 0) return KVARN_OK;
  if (block_pool == nullptr || src_blocks == nullptr || k_out == nullptr || v_out == nullptr)
    return KVARN_ERR_NULL_ARG;
  if (!aligned16(k_out) || !aligned16(v_out) || !aligned16(block_pool)) return KVARN_ERR_BAD_SHAPE;
  if (2LL * cfg->num_kv_heads * n_tiles > kMaxGrid) return KVARN_ERR_BAD_SHAPE;
  return from_hip(kvarn::launch_dequantize_tiles(static_cast<const uint8_t*>(block_pool),
                                                 num_blocks, src_blocks, n_tiles,
                                                 cfg->num_kv_heads, k_out, v_out,
                                                 cfg->rotation_signs, cfg->v_bits,
                                                 cfg->head_dim, static_cast<hipStream_t>(stream)));
}

// The unquantised comparison cache exists at head dimension 128 only.
static kvarn_status check_fp16_config(const kvarn_config* cfg) {
  const kvarn_status st = check_config(cfg);
  if (st != KVARN_OK) return st;
  return cfg->head_dim == KVARN_HEAD_DIM ? KVARN_OK : KVARN_ERR_UNSUPPORTED;
}

size_t kvarn_fp16_block_bytes(const kvarn_config* cfg) {
  return check_fp16_config(cfg) == KVARN_OK
             ? (size_t)KVARN_FP16_RECORD_BYTES * (size_t)cfg->num_kv_heads
             : 0;
}

kvarn_status kvarn_fp16_write_tiles(const kvarn_config* cfg, const void* k, const void* v,
                                    int64_t token_stride, int32_t n_tiles,
                                    const int32_t* dst_blocks, void* block_pool,
                                    int64_t num_blocks, void* stream) {
  kvarn_status st = check_fp16_config(cfg);
  if (st != KVARN_OK) return st;
  if (n_tiles < 0 || num_blocks < 0) return KVARN_ERR_BAD_SHAPE;
  if (n_tiles == 0) return KVARN_OK;
  if (k == nullptr || v == nullptr || dst_blocks == nullptr || block_pool == nullptr)
    return KVARN_ERR_NULL_ARG;
  if (token_stride < (int64_t)cfg->num_kv_heads * KVARN_HEAD_DIM || token_stride % 8 != 0 ||
      !aligned16(k) || !aligned16(v) || !aligned16(block_pool))
    return KVARN_ERR_BAD_SHAPE;
  if ((long long)cfg->num_kv_heads * n_tiles > kMaxGrid) return KVARN_ERR_BAD_SHAPE;
  return from_hip(kvarn::launch_fp16_write_tiles(
      static_cast<const __half*>(k), static_cast<const __half*>(v), token_stride, n_tiles,
      cfg->num_kv_heads, dst_blocks, static_cast<uint8_t*>(block_pool), num_blocks,
      static_cast<hipStream_t>(stream)));
}

kvarn_status kvarn_decode_attention_fp16(const kvarn_config* cfg, const void* q,
                                         int32_t num_q_heads, const void* block_pool,
                                         int64_t num_blocks, const int32_t* block_table,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                         const void* staging_k, const void* staging_v,
                                         float sm_scale, float* out, void* workspace,
                                         size_t workspace_bytes, int32_t batch, void* stream) {
  kvarn_status st = check_fp16_config(cfg);
  if (st != KVARN_OK) return st;
  size_t need = 0;
  st = kvarn_decode_workspace_bytes(cfg, batch, num_q_heads, max_blocks_per_seq, &need);
  if (st != KVARN_OK) return st;
  if (num_blocks < 0) return KVARN_ERR_BAD_SHAPE;
  if (batch == 0) return KVARN_OK;
  if (q == nullptr || block_pool == nullptr || block_table == nullptr || seq_lens == nullptr ||
      staging_k == nullptr || staging_v == nullptr || out == nullptr)
    return KVARN_ERR_NULL_ARG;
  if (workspace == nullptr || workspace_bytes < need) return KVARN_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KVARN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(staging_k) || !aligned16(staging_v) || !aligned16(out) ||
      !aligned16(block_pool))
    return KVARN_ERR_BAD_SHAPE;
  if (!(sm_scale == sm_scale)) return KVARN_ERR_BAD_SHAPE;
  if ((long long)batch > 65535 || cfg->num_kv_heads > 65535) return KVARN_ERR_BAD_SHAPE;
  const int splits = kvarn::decode_splits(batch, cfg->num_kv_heads, max_blocks_per_seq);
  if (workspace_bytes < (size_t)batch * (size_t)num_q_heads * (size_t)splits *
                            (size_t)kvarn::kPartialFloats * sizeof(float))
    return KVARN_ERR_WORKSPACE;                 // covered by the size above; checked anyway
  return from_hip(kvarn::launch_decode_fp16(
      static_cast<const __half*>(q), num_q_heads, cfg->num_kv_heads,
      static_cast<const uint8_t*>(block_pool), num_blocks, block_table, max_blocks_per_seq,
      seq_lens, static_cast<const __half*>(staging_k), static_cast<const __half*>(staging_v),
      sm_scale, out, static_cast<float*>(workspace), splits, batch,
      static_cast<hipStream_t>(stream)));
}

const char* kvarn_status_string(kvarn_status status) {
  switch (status) {
    case KVARN_OK: return "ok";
    case KVARN_ERR_NULL_ARG: return "a required pointer is NULL";
    case KVARN_ERR_BAD_SHAPE: return "a size or count is out of range, or a buffer is misaligned";
    case KVARN_ERR_UNSUPPORTED:
      return "unsupported config (k_bits 4, v_bits 2 or 4, block_tokens 128, head_dim 64, 128 "
             "or 256, sign words past head_dim / 32 zero; the fp16 cache: head_dim 128)";
    case KVARN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case KVARN_ERR_HIP: return "HIP runtime error while launching";
    case KVARN_ERR_SCRATCH_LIMIT:
      return "the decode needs more scratch than the library's static array "
             "(KVARN_STATIC_SCRATCH_BYTES); use kvarn_decode_attention with a workspace";
  }
  return "unknown status";
}

int32_t kvarn_abi_version(void) { return KVARN_ABI_VERSION; }

}  // extern "C"
