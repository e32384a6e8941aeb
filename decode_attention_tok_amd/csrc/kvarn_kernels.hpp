// Internal launch wrappers of the libkvarn kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kvarn {

// Floats per (sequence, query head, split) partial: m, l, rotated output (head dimension 128;
// 2 + head_dim in general).
constexpr int kPartialFloats = 2 + 128;
inline int partial_floats(int head_dim) { return 2 + head_dim; }
constexpr int kMaxGroup = 16;
constexpr int kMaxQuery = 16;        // query tokens per sequence in one multi-token decode

// v_bits: 2 (kvarn_k4v2_g128) or 4 (kvarn_k4v4_g128); head_dim: 64, 128 or 256. Together they
// fix the record size.
hipError_t launch_quantize_tiles(const __half* k, const __half* v, long long token_stride,
                                 int n_tiles, int hkv, const int32_t* dst_blocks,
                                 uint8_t* pool, long long num_blocks, int iters,
                                 const uint32_t* signs, int v_bits, int head_dim,
                                 hipStream_t stream);

hipError_t launch_append_token(const __half* k_new, const __half* v_new,
                               const int32_t* positions, const int32_t* block_table,
                               int max_blocks, __half* staging_k, __half* staging_v,
                               uint8_t* pool, long long num_blocks, int hkv, int batch,
                               int iters, const uint32_t* signs, int v_bits, int head_dim,
                               hipStream_t stream);

// nq query tokens per sequence (q, out: [batch][nq][hq][head_dim]); query token i sits at position
// len - nq + i and attends to positions 0 .. len - nq + i. nq = 1 is the one-token decode.
hipError_t launch_decode(const __half* q, int hq, int hkv, int nq, const uint8_t* pool,
                         long long num_blocks, const int32_t* block_table, int max_blocks,
                         const int32_t* seq_lens, const __half* staging_k,
                         const __half* staging_v, float sm_scale, float* out, float* partials,
                         int slots, int batch, const uint32_t* signs, int v_bits, int head_dim,
                         hipStream_t stream);

// signs: the eight words of optional per-channel sign flips before the rotation (host array;
// a head dimension d uses the first d / 32).

// Unquantised fp16 paged cache (comparison path): 65,536-byte record per (block, KV head).
constexpr long long kFp16RecordBytes = 65536;

hipError_t launch_fp16_write_tiles(const __half* k, const __half* v, long long token_stride,
                                   int n_tiles, int hkv, const int32_t* dst_blocks,
                                   uint8_t* pool, long long num_blocks, hipStream_t stream);

hipError_t launch_decode_fp16(const __half* q, int hq, int hkv, const uint8_t* pool,
                              long long num_blocks, const int32_t* block_table, int max_blocks,
                              const int32_t* seq_lens, const __half* staging_k,
                              const __half* staging_v, float sm_scale, float* out,
                              float* partials, int splits, int batch, hipStream_t stream);

// Records of blocks src_blocks[i] back to fp32 tiles in the original space: k_out, v_out
// [n_tiles * 128][hkv][head_dim]; invalid block ids give NaN rows.
hipError_t launch_dequantize_tiles(const uint8_t* pool, long long num_blocks,
                                   const int32_t* src_blocks, int n_tiles, int hkv, float* k_out,
                                   float* v_out, const uint32_t* signs, int v_bits, int head_dim,
                                   hipStream_t stream);

// Splits of each sequence's tiles for the split grid of the four-wave tile kernels (the fp16
// comparison decode, and packed decodes with several head groups per KV head): depends on the
// sizes and on the compute-unit count of the current device (read once per device and cached).
int decode_splits(int batch, int hkv, int max_blocks);
// Whether a decode of these sizes runs the paired-tile kernel (decode_pairs_kernel).
bool pairs_mode(int virtual_heads, int v_bits, int head_dim, int batch, int hkv, int max_blocks);
// The kernel and schedule of a packed decode (virtual heads = query heads per KV head x query
// tokens), and the partial slots per (sequence, query token, query head) row it needs.
enum class DecodeKind { kPairList, kWideList, kWideGrid, kTileList, kTileGrid };
DecodeKind decode_kind(int batch, int hkv, int max_blocks, int virtual_heads, int v_bits,
                       int head_dim);
int decode_slots(int batch, int hkv, int max_blocks, int virtual_heads, int v_bits,
                 int head_dim);
int device_compute_units();

}  // namespace kvarn
