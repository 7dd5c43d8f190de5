// Internal interface between the host-side API (pa_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum KvKind : int { KV_F32 = 0, KV_F16 = 1, KV_BF16 = 2, KV_FP8 = 3 };

// Everything a decode launch needs, already validated; strides in elements.
struct DecodeArgs {
  void *out;
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  float *ws_ml;   // [S, H, NP, 2] running max (log2 units) and sum per partition
  float *ws_acc;  // [S, H, NP, D] unnormalised partition outputs
  int64_t q_ss, q_sh;           // q strides: sequence, head
  int64_t o_ss, o_sh;           // out strides
  int64_t k_sb, k_st, k_sh;     // k_cache strides: block, token, kv head
  int64_t v_sb, v_st, v_sh;     // v_cache strides
  int64_t bt_ss;                // block-table row stride
  int32_t num_seqs, num_heads, num_kv_heads, head_dim;
  int32_t num_blocks, block_size, log2_block_size, max_blocks_per_seq;
  int32_t max_ctx;              // max_blocks_per_seq * block_size
  int32_t partition_size, num_partitions;
  float qk_scale_log2;          // scale * log2(e) (* k_scale for fp8)
  float v_scale;                // 1, or the fp8 value-cache scale
  int32_t kv_kind;              // KvKind
  int32_t q_kind;               // KV_F32 / KV_F16 / KV_BF16
  int32_t out_f32;              // 1: out is fp32, 0: out has q's dtype
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
};

// Launchers (defined in the .hip files).  They return the launch's hipError_t.
hipError_t launch_decode_partitions(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_cache_write(const CacheWriteArgs &a, hipStream_t stream);

// Which (kv dtype, q dtype, head_dim, group size) the decode kernels were built for.
bool decode_supported(int kv_kind, int q_kind, int head_dim, int group);

}  // namespace pa
