/*
 * kvarn.h - C ABI of libkvarn: the KVarN K4V2 g128 KV-cache codec (and a K4V4 variant) and
 * the paged decode attention that reads it, for AMD Instinct MI355X (gfx950).
 *
 * Sources. The operations follow these pages (cited by title and section):
 *   [GR]  groundy.com, "Huawei's KVarN puts KV-cache quantization inside vLLM's backend":
 *         "What KVarN changes in vLLM's serving path" (preset kvarn_k4v2_g128: 4-bit keys,
 *         2-bit values, one 128-token tile per cache block, FP8 scales and FP16 zero-points)
 *         and "The four-stage pipeline" (Hadamard rotation along channels; Sinkhorn-like
 *         alternating column/row standard-deviation normalisation in log space; asymmetric
 *         round-to-nearest; scales applied when a tile is read for attention), and
 *         "Frequently Asked Questions" (tile fixed at 128 tokens; the preset covers head
 *         dimension 128 only, and another geometry needs its own scale layout: head_dim 64
 *         and 256 are built here with the same stages and the layout below scaled with D).
 *   [TSM] tools.thesoundmethod.me, "KVarN: 2-Bit KV-Cache That Beats FP16 Throughput, and
 *         Where the Catch Lives", "What KVarN does differently" (the two conditioning steps)
 *         and "Where the bill lands" (rotation and per-tile statistics are state that must
 *         stay consistent between prefill and decode).
 *
 * Conventions shared by every entry point.
 *   - Pointers marked (device) are HIP device pointers; (host) are host pointers.
 *   - fp16 means IEEE binary16, little-endian. All fp16 buffers and every block pool must be
 *     16-byte aligned (a misaligned one gives KVARN_ERR_BAD_SHAPE).
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream. Every call
 *     validates its arguments on the host, then enqueues its kernels on `stream` and returns
 *     without synchronising. On a validation error nothing is enqueued.
 *   - The library allocates no device memory and keeps no state between calls; the caller
 *     owns every buffer. Calls on different buffers may run concurrently.
 *   - Every call only enqueues kernel launches (no allocation, no memset, no copy, no host
 *     synchronisation), so a sequence of calls on `stream` may be captured into a HIP graph
 *     and replayed; a replay computes what the captured calls compute on the buffers' contents
 *     at replay time. The decode's work split queries the device's compute-unit count and
 *     each kernel's occupancy on the host the first time they are needed, and caches them;
 *     make the same calls once before capturing, so that no query falls inside the capture.
 *   - Device-side preconditions that the host cannot see (block ids, positions, lengths) are
 *     bounds-checked in the kernels: an out-of-range block id or length never causes an
 *     out-of-bounds access; see each entry point for the result it then produces.
 *
 * The packed cache. A block holds 128 tokens of every KV head: num_kv_heads tile records of
 * R = kvarn_tile_bytes() bytes back to back (record of block b, KV head h at byte
 * (b * num_kv_heads + h) * R of the block pool). With head dimension D (head_dim) and
 * V = 16 D v_bits bytes of value codes, R = 64 D + V + 2 (D + 384): 13312 for the preset
 * kvarn_k4v2_g128 (D = 128, v_bits 2) and 17408 for kvarn_k4v4_g128 (v_bits 4); 7040 and
 * 9088 at D = 64; 25856 and 34048 at D = 256. A record, little-endian, with K = 64 D and
 * M = K + V:
 *   [0, K)         key codes (4 bit), token-major: token t at byte (D / 2) t; channel j in
 *                  byte j / 2, low nibble for even j, high nibble for odd j
 *   [K, M)         value codes, as 32-bit words. With nb = j / 16, n = j % 16, kb = t / 32,
 *                  h = (t / 16) % 2, s = (t / 4) % 4, i = t % 4 and e = 2 h + i / 2, the
 *                  code of token t, channel j is at
 *                    v_bits 2, D >= 128: word 2 D kb + (D / 32)(16 s + n) + 4 (nb / 8) + e,
 *                              bits 2 (nb % 8) + 16 (i % 2) .. +1
 *                    v_bits 2, D = 64: word 128 kb + 2 (16 s + n) + e / 2,
 *                              bits 2 nb + 8 (e % 2) + 16 (i % 2) .. +1
 *                    v_bits 4: word 4 D kb + 256 (nb / 4) + 4 (16 s + n) + e,
 *                              bits 4 (nb % 4) + 16 (i % 2) .. +3
 *   [M, M + D)               key per-channel scale c-hat, FP8 E4M3 (OCP), channel j at byte j
 *   [M + D, M + D + 128)     key per-token scale s-hat, FP8 E4M3, token t at byte t
 *   [M + D + 128, M + D + 384) key per-token zero-point z-hat, fp16, token t at bytes 2t, 2t+1
 *   [M + D + 384, R)         the same three arrays for the values
 * (D = 128: key codes [0, 8192), value codes from 8192, metadata halves of 512 bytes.)
 * A dequantised rotated element is c-hat_j * (s-hat_t * code_tj + z-hat_t); the original
 * element is the rotated row times the D-point orthonormal Sylvester Hadamard matrix.
 *
 * The fp16 staging tile. Tokens past the last full block of a sequence live unquantised in
 * staging[b][h][t][0..D-1] (fp16, [batch][num_kv_heads][128][D]): a sequence of L tokens
 * reads floor(L / 128) packed tiles through its block-table row and L mod 128 staging
 * tokens. kvarn_append_token fills staging and quantises it when it holds 128 tokens; a
 * prefill tail may also be written there directly in this plain layout.
 */
#ifndef KVARN_H
#define KVARN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define KVARN_API __attribute__((visibility("default")))
#else
#define KVARN_API
#endif

#define KVARN_ABI_VERSION 5
#define KVARN_TILE_TOKENS 128
#define KVARN_HEAD_DIM 128            /* the preset's; 64 and 256 are accepted too */
#define KVARN_SIGN_WORDS 8
#define KVARN_TILE_BYTES 13312        /* record of the default preset (v_bits 2) */
#define KVARN_TILE_BYTES_V4 17408     /* record with v_bits 4 (head_dim 128)     */
#define KVARN_FP16_RECORD_BYTES 65536

typedef enum {
  KVARN_OK = 0,
  KVARN_ERR_NULL_ARG = 1,    /* a required pointer is NULL                               */
  KVARN_ERR_BAD_SHAPE = 2,   /* a size or count is out of range, or a buffer misaligned  */
  KVARN_ERR_UNSUPPORTED = 3, /* the config is not one of the presets below                */
  KVARN_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required               */
  KVARN_ERR_HIP = 5,         /* the HIP runtime reported an error when launching         */
  KVARN_ERR_SCRATCH_LIMIT = 6 /* kvarn_decode_attention_noalloc: sizes beyond its scratch  */
} kvarn_status;

/* The codec configuration. The pages ship one preset, kvarn_k4v2_g128 ([GR], "What KVarN
 * changes in vLLM's serving path" and "Frequently Asked Questions"): head_dim 128,
 * block_tokens 128, k_bits 4, v_bits 2 (the default). v_bits 4 selects a second preset,
 * kvarn_k4v4_g128, not on the pages: the same four stages with 4-bit value codes on a grid of
 * 16 levels ([GR] "The four-stage pipeline", stage 3, at another bit width) and a 17408-byte
 * record. head_dim 64 or 256 runs the same stages on 128-token tiles of that many channels
 * (a D-point rotation, D per-channel scales, the same rounds and floor; [GR] "Frequently
 * Asked Questions" leaves other geometries open). sinkhorn_iters is the fixed number of
 * column+row normalisation rounds of [GR] "The four-stage pipeline" stage 2, whose value the
 * pages do not give: 4 by default, 1..16 accepted. Prefill and decode must use the same
 * config ([TSM] "Where the bill lands"). */
typedef struct {
  int32_t num_kv_heads;   /* >= 1                      */
  int32_t head_dim;       /* 64, 128 (default) or 256  */
  int32_t block_tokens;   /* must be 128               */
  int32_t k_bits;         /* must be 4                 */
  int32_t v_bits;         /* 2 (default) or 4          */
  int32_t sinkhorn_iters; /* 1..16, default 4          */
  /* Optional sign flips before the rotation (a randomised-sign Hadamard; not part of the
   * pages' preset): channel j is negated before H when bit j % 32 of rotation_signs[j / 32]
   * is set, and again after H on the read path. All zero (the default) is the plain
   * Hadamard of the preset. Words from head_dim / 32 on must be zero. Records written with
   * one setting must be read with the same. */
  uint32_t rotation_signs[KVARN_SIGN_WORDS];
} kvarn_config;

/* Fills *cfg with the preset for num_kv_heads heads (sinkhorn_iters = 4, no sign flips). */
KVARN_API void kvarn_default_config(kvarn_config* cfg, int32_t num_kv_heads);

/* Bytes of one tile record (one KV head of one block, keys and values): 64 D + 16 D v_bits +
 * 2 (D + 384) for head dimension D (13312 for v_bits 2 and 17408 for v_bits 4 at D = 128),
 * or 0 if the config is invalid. */
KVARN_API size_t kvarn_tile_bytes(const kvarn_config* cfg);

/* Bytes of one block: num_kv_heads * kvarn_tile_bytes, or 0 if the config is invalid. */
KVARN_API size_t kvarn_block_bytes(const kvarn_config* cfg);

/* Write path, prefill ([GR] "The four-stage pipeline", stages 1-3, per 128-token tile).
 * Quantises n_tiles whole tiles of keys and values into the block pool.
 *   k, v          (device) fp16, token-major: token i of the input, KV head h, channel j at
 *                 element i * token_stride + h * D + j (D = head_dim), for i < n_tiles * 128.
 *                 Tile m is tokens 128 m .. 128 m + 127.
 *   token_stride  elements between consecutive tokens; >= num_kv_heads * D, multiple of 8.
 *   dst_blocks    (device) int32 [n_tiles]: tile m is written to block dst_blocks[m].
 *   block_pool    (device) num_blocks blocks of kvarn_block_bytes.
 * n_tiles = 0 is a no-op. A dst_blocks entry outside [0, num_blocks) skips that tile.
 * Two tiles with the same destination race. */
KVARN_API kvarn_status kvarn_quantize_tiles(const kvarn_config* cfg, const void* k, const void* v,
                                  int64_t token_stride, int32_t n_tiles,
                                  const int32_t* dst_blocks, void* block_pool,
                                  int64_t num_blocks, void* stream);

/* Write path, one decode step ([GR] "The four-stage pipeline", stage 4: a token's write does
 * no dequantisation work). For each sequence b with positions[b] >= 0, writes its new key and value
 * token into staging slot positions[b] % 128; when that slot is 127 the staging tile now
 * holds 128 tokens and is quantised into block block_table[b][positions[b] / 128].
 *   k_new, v_new      (device) fp16 [batch][num_kv_heads][D]
 *   positions         (device) int32 [batch]: 0-based index of the new token; < 0 skips
 *   block_table       (device) int32 [batch][max_blocks_per_seq]
 *   staging_k/_v      (device) fp16 [batch][num_kv_heads][128][D], updated in place
 *   block_pool        (device) num_blocks blocks
 * If positions[b] / 128 >= max_blocks_per_seq or the block id is outside [0, num_blocks),
 * the staging write still happens and the completed tile is not quantised. */
KVARN_API kvarn_status kvarn_append_token(const kvarn_config* cfg, const void* k_new, const void* v_new,
                                const int32_t* positions, const int32_t* block_table,
                                int32_t max_blocks_per_seq, void* staging_k, void* staging_v,
                                void* block_pool, int64_t num_blocks, int32_t batch,
                                void* stream);

/* Size of the workspace kvarn_decode_attention needs for these sizes, into *bytes (host).
 * It depends on the arguments and on the compute-unit count of the current HIP device (the
 * work is planned for the device's compute units; 256 are assumed when no device is usable),
 * so query it with the device current that will run the decode. It holds one partial result
 * of 2 + head_dim floats per query head and partial slot: the slots of a sequence's tiles
 * are at most 64, from the table width alone (the actual lengths are read on the device).
 * The same size also serves kvarn_decode_attention_fp16 at these sizes. */
KVARN_API kvarn_status kvarn_decode_workspace_bytes(const kvarn_config* cfg, int32_t batch,
                                          int32_t num_q_heads, int32_t max_blocks_per_seq,
                                          size_t* bytes);

/* Read path ([GR] "The four-stage pipeline", stage 4, with stage 1's rotation folded into
 * the query and the output). Exact softmax attention of one query token per (sequence,
 * query head) over floor(L/128) dequantised packed tiles and L mod 128 fp16 staging tokens,
 * L = seq_lens[b]. Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *   q            (device) fp16 [batch][num_q_heads][D]; num_q_heads a multiple of
 *                num_kv_heads with num_q_heads / num_kv_heads <= 16
 *   block_pool   (device) num_blocks blocks
 *   block_table  (device) int32 [batch][max_blocks_per_seq]
 *   seq_lens     (device) int32 [batch]
 *   staging_k/_v (device) fp16 [batch][num_kv_heads][128][D]
 *   sm_scale     softmax scale applied to q . k (for example 1/sqrt(D))
 *   out          (device) fp32 [batch][num_q_heads][D]
 *   workspace    (device) at least kvarn_decode_workspace_bytes bytes, 256-byte aligned;
 *                its contents on entry do not matter
 * L = 0 gives zeros. A row with L < 0, L / 128 > max_blocks_per_seq or a block id outside
 * [0, num_blocks) gives NaN in every output of that sequence. */
KVARN_API kvarn_status kvarn_decode_attention(const kvarn_config* cfg, const void* q, int32_t num_q_heads,
                                    const void* block_pool, int64_t num_blocks,
                                    const int32_t* block_table, int32_t max_blocks_per_seq,
                                    const int32_t* seq_lens, const void* staging_k,
                                    const void* staging_v, float sm_scale, float* out,
                                    void* workspace, size_t workspace_bytes, int32_t batch,
                                    void* stream);

/* Stage 4 written out ([GR] "The four-stage pipeline": dequantisation restores each element
 * from its code, the per-token scale and zero-point and the per-channel scale, and the
 * rotation is undone): the records of blocks src_blocks[i] back to fp32 tiles in the original
 * channel space, for inspection, export and error measurement (decode attention never does
 * this; it folds the same arithmetic into the scores and outputs).
 *   src_blocks  (device) int32 [n_tiles]; an id outside [0, num_blocks) gives NaN rows
 *   k_out,v_out (device) fp32 [n_tiles * 128][num_kv_heads][D], 16-byte aligned: token
 *               128 i + t of KV head h from record (src_blocks[i], h)
 * Errors: NULL_ARG, BAD_SHAPE (negative counts, misaligned outputs or pool, too many tiles). */
KVARN_API kvarn_status kvarn_dequantize_tiles(const kvarn_config* cfg, const void* block_pool,
                                    int64_t num_blocks, const int32_t* src_blocks,
                                    int32_t n_tiles, float* k_out, float* v_out, void* stream);

/* ---- Decode without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The library keeps
 * one static device array of KVARN_STATIC_SCRATCH_BYTES per GPU it runs on (held until the
 * process ends) and uses it as the workspace of kvarn_decode_attention; the call itself
 * allocates nothing. Every call on one GPU shares that GPU's array, so calls that overlap on
 * one GPU (different streams, or different threads) race and must not be issued; the array
 * needs no clearing (the decode writes every partial it reads). Arguments, results, NaN rules
 * and errors are those of kvarn_decode_attention without the workspace, plus
 * KVARN_ERR_SCRATCH_LIMIT when kvarn_decode_workspace_bytes for these sizes exceeds
 * KVARN_STATIC_SCRATCH_BYTES (nothing is launched then), and KVARN_ERR_HIP if the array's
 * device address cannot be obtained. */
#define KVARN_STATIC_SCRATCH_BYTES (16u << 20)

KVARN_API kvarn_status kvarn_decode_attention_noalloc(const kvarn_config* cfg, const void* q,
                                            int32_t num_q_heads, const void* block_pool,
                                            int64_t num_blocks, const int32_t* block_table,
                                            int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                            const void* staging_k, const void* staging_v,
                                            float sm_scale, float* out, int32_t batch,
                                            void* stream);

/* ---- Several query tokens per sequence (multi-token verification, chunked continuation).
 * The pages place KVarN beside speculative decoding and multi-token prediction ([GR] "The 2-bit
 * quantization field"); those steps score Q new tokens per sequence at once. Reading taken
 * here: the Q tokens are the last Q of the sequence's L = seq_lens[b] tokens, already written
 * to the cache (kvarn_append_token once per token), and query token i (0-based) sits at
 * position L - Q + i and attends to positions 0 .. L - Q + i (causal); an empty range gives
 * zeros. Q = 1 is exactly kvarn_decode_attention. */
#define KVARN_MAX_QUERY_TOKENS 16

/* Workspace for kvarn_decode_attention_multi (host), as kvarn_decode_workspace_bytes;
 * KVARN_ERR_BAD_SHAPE unless 1 <= n_query <= KVARN_MAX_QUERY_TOKENS. */
KVARN_API kvarn_status kvarn_decode_multi_workspace_bytes(const kvarn_config* cfg, int32_t batch,
                                                int32_t num_q_heads, int32_t n_query,
                                                int32_t max_blocks_per_seq, size_t* bytes);

/* kvarn_decode_attention for n_query tokens per sequence:
 *   q    (device) fp16 [batch][n_query][num_q_heads][D]
 *   out  (device) fp32 [batch][n_query][num_q_heads][D]
 *   workspace at least kvarn_decode_multi_workspace_bytes bytes, 256-byte aligned
 * Every other argument, the NaN rules and the errors as kvarn_decode_attention. */
KVARN_API kvarn_status kvarn_decode_attention_multi(const kvarn_config* cfg, const void* q,
                                          int32_t num_q_heads, int32_t n_query,
                                          const void* block_pool, int64_t num_blocks,
                                          const int32_t* block_table, int32_t max_blocks_per_seq,
                                          const int32_t* seq_lens, const void* staging_k,
                                          const void* staging_v, float sm_scale, float* out,
                                          void* workspace, size_t workspace_bytes, int32_t batch,
                                          void* stream);

/* ---- Unquantised fp16 paged cache: the comparison path. The pages compare KVarN with FP16
 * serving of the same model ([GR] "Reported benchmarks and the verification gap"); these
 * calls give the same decode over an fp16 cache with the same paging, staging and GQA
 * rules, so the two can be measured on the same shapes. Record of one (block, KV head):
 * KVARN_FP16_RECORD_BYTES = 65,536 bytes, keys first as fp16 [token][channel] (32,768 B),
 * then values as fp16 [channel][position] (32,768 B), where position 32 kb + 8 s + e of a
 * row holds token 32 kb + 16 (e / 4) + 4 s + e % 4 (kb, s in 0..3, e in 0..7). A block is
 * num_kv_heads records, head-major, like the packed pool. These calls take head_dim 128 only
 * (KVARN_ERR_UNSUPPORTED otherwise). */

/* Bytes of one fp16 block: num_kv_heads * 65536, or 0 if the config is invalid. */
KVARN_API size_t kvarn_fp16_block_bytes(const kvarn_config* cfg);

/* Write whole tiles into the fp16 pool: the counterpart of kvarn_quantize_tiles, same
 * arguments, layout rules and errors (k, v fp16 [n_tiles * 128][token_stride], tile i to
 * block dst_blocks[i]; ids outside [0, num_blocks) are skipped); block_pool holds num_blocks
 * fp16 blocks. */
KVARN_API kvarn_status kvarn_fp16_write_tiles(const kvarn_config* cfg, const void* k, const void* v,
                                    int64_t token_stride, int32_t n_tiles,
                                    const int32_t* dst_blocks, void* block_pool,
                                    int64_t num_blocks, void* stream);

/* Exact softmax attention over the fp16 pool: the counterpart of kvarn_decode_attention, same
 * arguments (block_pool holds fp16 blocks), workspace size (kvarn_decode_workspace_bytes),
 * NaN rules and errors. */
KVARN_API kvarn_status kvarn_decode_attention_fp16(const kvarn_config* cfg, const void* q,
                                         int32_t num_q_heads, const void* block_pool,
                                         int64_t num_blocks, const int32_t* block_table,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                         const void* staging_k, const void* staging_v,
                                         float sm_scale, float* out, void* workspace,
                                         size_t workspace_bytes, int32_t batch, void* stream);

/* Static, NUL-terminated description of a status. */
KVARN_API const char* kvarn_status_string(kvarn_status status);

/* KVARN_ABI_VERSION of the built library. */
KVARN_API int32_t kvarn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVARN_H */
