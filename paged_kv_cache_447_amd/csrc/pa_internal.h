// Internal interface between the host-side API (pa_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum KvKind : int { KV_F32 = 0, KV_F16 = 1, KV_BF16 = 2, KV_FP8 = 3 };

// Everything a decode launch needs, already validated; strides in elements.
//
// Work decomposition (shared by every decode kernel): the context of each
// (sequence, kv head) pair -- an "item" -- is cut into units of part_tokens
// tokens.  Items are ordered sequence-major, then kv head, then unit, and the
// num_workers wavefronts of the launch each take one contiguous, equally sized
// range of that order.  A worker whose range covers a whole item writes the
// item's output; a range that cuts an item leaves a partial result (running
// max, running sum, unnormalised output) in one of its two workspace slots,
// and the last worker to finish an item merges the partials by log-sum-exp.
struct DecodeArgs {
  void *out;
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  int32_t *counters;   // [S * Hkv] finished-partial counters; zero between calls
  float *part_ml;      // [2 * num_workers, G, 2] partial (max in log2 units, sum)
  float *part_acc;     // [2 * num_workers, G, D] partial unnormalised outputs
  uint32_t ml_bytes, acc_bytes;  // sizes of the two partial regions (< 2^32)
  int64_t q_ss, q_sh;           // q strides: sequence, head
  int64_t o_ss, o_sh;           // out strides
  int64_t k_sb, k_st, k_sh;     // k_cache strides: block, token, kv head
  int64_t v_sb, v_st, v_sh;     // v_cache strides
  int64_t bt_ss;                // block-table row stride
  int32_t num_seqs, num_heads, num_kv_heads, head_dim;
  int32_t num_blocks, block_size, max_blocks_per_seq;
  int32_t max_ctx;              // max_blocks_per_seq * block_size
  int32_t part_tokens;          // tokens per work unit
  int32_t num_workers;          // wavefronts in the launch
  float qk_scale_log2;          // scale * log2(e) (* k_scale for fp8)
  float v_scale;                // 1, or the fp8 value-cache scale
  // fp8 caches with one scale per (layer, kv head): [layers * num_kv_heads]
  // each, multiplied into the two above (then scale * log2(e) and 1); or null
  const float *k_head_scale, *v_head_scale;
  // fp8 caches with one scale per (layer, block, kv head): [layers *
  // num_blocks * num_kv_heads] each, the scale of a token's block applied to
  // its score (key) and its weight (value); or null
  const float *k_block_scale, *v_block_scale;
  int32_t kv_kind;              // KvKind
  int32_t q_kind;               // KV_F32 / KV_F16 / KV_BF16
  int32_t out_f32;              // 1: out is fp32, 0: out has q's dtype
  // Several layers in one launch: sequence s of the launch is sequence
  // s % seqs_per_layer of layer s / seqs_per_layer.  The layers share the block
  // tables and context lengths; each has its own query, output and caches, at
  // these strides (elements).  One layer: seqs_per_layer = num_seqs.
  int32_t seqs_per_layer;
  int64_t q_sl, o_sl, k_sl, v_sl;
  // pa_decode_append: the step's new token of every sequence, stored at its
  // slot by the launch itself and read in place of the cache row at position
  // context_len - 1 (one layer; the new rows have the cache's dtype)
  int32_t append;
  const void *k_new, *v_new;       // [num_seqs, num_kv_heads, head_dim]
  int64_t kn_ss, kn_sh, vn_ss, vn_sh;
  const void *slot_mapping;        // [num_seqs] int32 or int64
  int32_t slot_i64;
  int64_t num_slots;               // num_blocks * block_size
};

// Everything a prefill launch needs, already validated; strides in elements.
// Query rows qsl[s] .. qsl[s+1]-1 belong to sequence s and are its newest
// tokens: row j of n sits at position context_len - n + j and sees the
// positions up to its own.  The (row, query head) pairs of a sequence and kv
// head -- its "columns", row-major, G heads per row -- are cut into tiles of a
// fixed number of columns; one workgroup computes one tile.
struct PrefillArgs {
  void *out;
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *query_start_loc;  // [S + 1]
  int64_t q_sn, q_sh;              // q strides: row, head
  int64_t o_sn, o_sh;              // out strides
  int64_t k_sb, k_st, k_sh;        // k_cache strides: block, token, kv head
  int64_t v_sb, v_st, v_sh;        // v_cache strides
  int64_t bt_ss;                   // block-table row stride
  int32_t num_seqs, num_rows, num_heads, num_kv_heads, group, head_dim;
  int32_t num_blocks, block_size, max_ctx;
  int32_t tile_slots;              // tile slots per kv head in the grid (>= the tiles of all sequences)
  int32_t tile_cols;               // columns per tile
  int32_t key_split;               // 1: the four wavefronts split a tile's keys, 0: its columns
  int32_t persistent_wgs;          // key split: workgroups of the persistent launch (one per CU)
  int32_t *pair_counter;           // key split: pairs handed out so far (zero between calls), or null:
                                   // the pairs are then dealt round-robin
  float qk_scale_log2;             // scale * log2(e) (* k_scale for fp8)
  float v_scale;                   // 1, or the fp8 value-cache scale
  // fp8 caches with one scale per kv head: [num_kv_heads] each, multiplied
  // into the two above (then scale * log2(e) and 1); or null
  const float *k_head_scale, *v_head_scale;
  const float *k_block_scale, *v_block_scale;  // fp8 caches: [num_blocks * num_kv_heads] each, or null
  int32_t kv_kind;                 // KvKind of the caches: q's, or KV_FP8
  int32_t q_kind;                  // KvKind of q (and of the matrix-core operands)
  int32_t out_f32;                 // 1: out is fp32, 0: out has q's dtype
};

// Whole-block copies between two pools (copy-on-write, swap): for every pair
// (s, d) of the mapping, the K and V bytes of source block s become those of
// destination block d.  Pointers are device addresses (of device memory or of
// pinned, device-mapped host memory).
struct BlockCopyArgs {
  char *dst_k, *dst_v;
  const char *src_k, *src_v;
  const void *mapping;           // [num_pairs, 2] (source, destination)
  int32_t map_i64;               // 1: int64 pairs, 0: int32
  int64_t map_stride;            // elements between consecutive pairs
  int64_t num_pairs;
  int64_t block_bytes;           // bytes of one block, contiguous in both pools
  int64_t src_stride, dst_stride;  // bytes between consecutive blocks
  int64_t src_blocks, dst_blocks;
  int32_t pieces;                // workgroups per (pair, K or V)
};

struct CacheWriteArgs {
  const void *k;
  const void *v;
  void *k_cache;
  void *v_cache;
  const void *slot_mapping;
  int32_t slot_i64;
  int64_t k_sn, k_sh, v_sn, v_sh;  // input strides: token, head
  int64_t kc_sb, kc_st, kc_sh;     // k_cache strides
  int64_t vc_sb, vc_st, vc_sh;     // v_cache strides
  int32_t num_tokens, num_kv_heads, head_dim;
  int64_t num_slots;               // num_blocks * block_size
  int32_t block_size;
  int32_t in_kind, cache_kind;     // KvKind of the inputs and of the cache
  float k_scale, v_scale;          // fp8 caches only
  const float *k_head_scale, *v_head_scale;  // fp8 caches: [num_kv_heads] each, or null (per-tensor scales)
  const float *k_block_scale, *v_block_scale;  // fp8 caches: [num_blocks * num_kv_heads] each, or null
};

// Tokens per chunk (the unit of one pipelined load batch) of the decode kernel
// that serves this configuration; work units are multiples of it by default.
int decode_chunk_tokens(int kv_kind, int head_dim, int group);

// Launchers (defined in the .hip files).  They return the launch's hipError_t.
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
// grouped-query heads on the matrix cores (decode_mfma.hip)
bool decode_uses_mfma(int kv_kind, int head_dim, int group);
int decode_mfma_chunk_tokens();
hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_cache_write(const CacheWriteArgs &a, hipStream_t stream);
// causal multi-token queries on the matrix cores (prefill_mfma.hip)
bool prefill_supported(int kv_kind, int head_dim);
void prefill_plan(int64_t num_rows, int64_t num_seqs, int group, int &tile_cols, int &key_split);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);
// whole-block copies (block_copy.hip)
int64_t copy_blocks_pieces(int64_t block_bytes);
hipError_t launch_copy_blocks(const BlockCopyArgs &a, hipStream_t stream);
// a plain streaming read, for measurement (stream_read.hip)
hipError_t launch_stream_read(const void *buf, int64_t bytes, int workgroups, int loads, bool nontemporal,
                              uint32_t *partials, hipStream_t stream);

// Which (kv dtype, q dtype, head_dim, group size) the decode kernels were built for.
bool decode_supported(int kv_kind, int q_kind, int head_dim, int group);

}  // namespace pa
