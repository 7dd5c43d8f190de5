// Host side of the C ABI declared in include/pa.h: argument validation, the
// partition-size choice, workspace carving and kernel dispatch.  Nothing here
// allocates device memory or waits for the device.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "pa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

pa_status fail(pa_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

int elem_bytes(int32_t dt) {
  switch (dt) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    case PA_FP8_E4M3: return 1;
    case PA_I32: return 4;
    case PA_I64: return 8;
  }
  return 0;
}

int kv_kind(int32_t dt) {
  switch (dt) {
    case PA_F32: return pa::KV_F32;
    case PA_F16: return pa::KV_F16;
    case PA_BF16: return pa::KV_BF16;
    case PA_FP8_E4M3: return pa::KV_FP8;
  }
  return -1;
}

// rank, non-null data, contiguous last dimension, 16-byte alignment of the base
// and of every outer stride (vector loads/stores address whole rows)
// (an empty tensor may have a NULL data pointer)
pa_status check_tensor(const pa_tensor &t, const char *name, int ndim, bool need_rows_aligned) {
  if (t.ndim != ndim) return fail(PA_ERR_SHAPE, "%s: rank %d, expected %d", name, t.ndim, ndim);
  const int eb = elem_bytes(t.dtype);
  if (!eb) return fail(PA_ERR_DTYPE, "%s: unknown dtype %d", name, t.dtype);
  bool empty = false;
  for (int i = 0; i < ndim; ++i) {
    if (t.shape[i] < 0) return fail(PA_ERR_SHAPE, "%s: negative size in dim %d", name, i);
    empty = empty || t.shape[i] == 0;
  }
  if (empty) return PA_OK;
  if (!t.data) return fail(PA_ERR_NULL, "%s: data pointer is NULL", name);
  if (t.stride[ndim - 1] != 1 && t.shape[ndim - 1] > 1)
    return fail(PA_ERR_LAYOUT, "%s: last dimension must be contiguous", name);
  if (need_rows_aligned) {
    if (reinterpret_cast<uintptr_t>(t.data) % 16)
      return fail(PA_ERR_LAYOUT, "%s: data pointer not 16-byte aligned", name);
    for (int i = 0; i < ndim - 1; ++i)
      if ((t.stride[i] * eb) % 16 && t.shape[i] > 1)
        return fail(PA_ERR_LAYOUT, "%s: stride of dim %d is not a multiple of 16 bytes", name, i);
  }
  return PA_OK;
}

int32_t choose_partition(int64_t num_seqs, int64_t num_kv_heads, int64_t max_blocks, int32_t block_size) {
  // Split long contexts until (sequence, kv head, partition) work items
  // comfortably outnumber the 256 compute units, but never below 256 tokens.
  const int64_t max_ctx = max_blocks * block_size;
  const int64_t pairs = num_seqs * num_kv_heads > 0 ? num_seqs * num_kv_heads : 1;
  int64_t p = 256;
  while (p < 4096 && pairs * ((max_ctx + p - 1) / p) > 16384) p *= 2;
  if (p < block_size) p = block_size;
  return (int32_t)p;
}

}  // namespace

extern "C" {

int32_t pa_decode_partition_size(int64_t num_seqs, int64_t num_kv_heads, int64_t max_blocks_per_seq,
                                 int32_t block_size) {
  if (block_size <= 0 || max_blocks_per_seq < 0) return 0;
  return choose_partition(num_seqs, num_kv_heads, max_blocks_per_seq, block_size);
}

size_t pa_decode_workspace_size(int64_t num_seqs, int64_t num_heads, int64_t num_kv_heads, int64_t head_dim,
                                int64_t max_blocks_per_seq, int32_t block_size, int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 ||
      block_size <= 0)
    return 0;
  const int64_t p =
      partition_size > 0 ? partition_size : choose_partition(num_seqs, num_kv_heads, max_blocks_per_seq, block_size);
  const int64_t np = (max_blocks_per_seq * block_size + p - 1) / p;
  if (np <= 1) return 0;
  const int64_t rows = num_seqs * num_heads * np;
  return (size_t)(rows * 2 + rows * head_dim) * sizeof(float);
}

pa_status pa_decode(pa_tensor out, pa_tensor q, pa_tensor k_cache, pa_tensor v_cache, pa_tensor block_tables,
                    pa_tensor context_lens, int32_t block_size, float scale, int32_t num_kv_heads,
                    const pa_opts *opts) {
  pa_opts o;
  std::memset(&o, 0, sizeof o);
  if (opts) o = *opts;
  pa_status st;
  if ((st = check_tensor(out, "out", 3, true))) return st;
  if ((st = check_tensor(q, "q", 3, true))) return st;
  if ((st = check_tensor(k_cache, "k_cache", 4, true))) return st;
  if ((st = check_tensor(v_cache, "v_cache", 4, true))) return st;
  if ((st = check_tensor(block_tables, "block_tables", 2, false))) return st;
  if ((st = check_tensor(context_lens, "context_lens", 1, false))) return st;

  if (q.dtype != PA_F32 && q.dtype != PA_F16 && q.dtype != PA_BF16)
    return fail(PA_ERR_DTYPE, "q: dtype must be F32, F16 or BF16");
  if (k_cache.dtype != v_cache.dtype) return fail(PA_ERR_DTYPE, "k_cache and v_cache dtypes differ");
  const int kvk = kv_kind(k_cache.dtype);
  if (kvk < 0) return fail(PA_ERR_DTYPE, "k_cache: dtype must be F32, F16, BF16 or FP8_E4M3");
  if (kvk == pa::KV_FP8 ? q.dtype == PA_F32 : k_cache.dtype != q.dtype)
    return fail(PA_ERR_DTYPE, "q dtype must equal the cache dtype (F16 or BF16 for an FP8 cache)");
  if (out.dtype != q.dtype && out.dtype != PA_F32) return fail(PA_ERR_DTYPE, "out: dtype must be q's dtype or F32");
  if (block_tables.dtype != PA_I32) return fail(PA_ERR_DTYPE, "block_tables: dtype must be I32");
  if (context_lens.dtype != PA_I32) return fail(PA_ERR_DTYPE, "context_lens: dtype must be I32");

  const int64_t S = q.shape[0], H = q.shape[1], D = q.shape[2];
  const int64_t NB = k_cache.shape[0];
  for (int i = 0; i < 3; ++i)
    if (out.shape[i] != q.shape[i]) return fail(PA_ERR_SHAPE, "out shape differs from q shape in dim %d", i);
  for (int i = 0; i < 4; ++i)
    if (k_cache.shape[i] != v_cache.shape[i]) return fail(PA_ERR_SHAPE, "k_cache and v_cache shapes differ");
  if (k_cache.shape[1] != block_size)
    return fail(PA_ERR_SHAPE, "block_size %d != k_cache.shape[1] %lld", block_size, (long long)k_cache.shape[1]);
  if (k_cache.shape[2] != num_kv_heads)
    return fail(PA_ERR_SHAPE, "num_kv_heads %d != k_cache.shape[2] %lld", num_kv_heads, (long long)k_cache.shape[2]);
  if (k_cache.shape[3] != D) return fail(PA_ERR_SHAPE, "k_cache head_dim %lld != q head_dim %lld",
                                         (long long)k_cache.shape[3], (long long)D);
  if (num_kv_heads <= 0 || H % num_kv_heads) return fail(PA_ERR_SHAPE, "num_heads %lld not a multiple of num_kv_heads %d",
                                                         (long long)H, num_kv_heads);
  if (block_tables.shape[0] != S) return fail(PA_ERR_SHAPE, "block_tables has %lld rows, q has %lld sequences",
                                              (long long)block_tables.shape[0], (long long)S);
  if (context_lens.shape[0] != S) return fail(PA_ERR_SHAPE, "context_lens has %lld entries, q has %lld sequences",
                                              (long long)context_lens.shape[0], (long long)S);
  if (block_size != 16 && block_size != 32) return fail(PA_ERR_UNSUPPORTED, "block_size %d (built: 16, 32)", block_size);
  if (!pa::decode_supported(kvk, kv_kind(q.dtype), (int)D, (int)(H / num_kv_heads)))
    return fail(PA_ERR_UNSUPPORTED, "no kernel for head_dim %lld, group size %lld with these dtypes "
                "(built: head_dim 64/128, group 1/2/4/8)", (long long)D, (long long)(H / num_kv_heads));
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(PA_ERR_ARG, "scale must be finite and > 0");
  float ks = o.k_scale == 0.0f ? 1.0f : o.k_scale, vs = o.v_scale == 0.0f ? 1.0f : o.v_scale;
  if (kvk != pa::KV_FP8) ks = vs = 1.0f;
  if (!(ks > 0.0f) || !std::isfinite(ks) || !(vs > 0.0f) || !std::isfinite(vs))
    return fail(PA_ERR_ARG, "k_scale / v_scale must be finite and > 0");
  if (o.flags != 0) return fail(PA_ERR_ARG, "flags must be 0");
  const int64_t W = block_tables.shape[1];
  if (S > 65535 || num_kv_heads > 65535) return fail(PA_ERR_UNSUPPORTED, "more than 65535 sequences or kv heads");
  if (W * block_size > (int64_t)1 << 30) return fail(PA_ERR_UNSUPPORTED, "table width too large");
  if (NB > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "more than 2^31-1 blocks");
  if (S == 0 || H == 0) return PA_OK;
  if (NB == 0 || W == 0) return fail(PA_ERR_SHAPE, "empty cache or block table");

  int64_t part = o.partition_size ? o.partition_size : choose_partition(S, num_kv_heads, W, block_size);
  if (part <= 0 || part % block_size) return fail(PA_ERR_ARG, "partition_size %lld must be a positive multiple of "
                                                  "block_size", (long long)part);
  const int64_t max_ctx = W * block_size;
  if (part > max_ctx) part = ((max_ctx + block_size - 1) / block_size) * block_size;
  const int64_t np = (max_ctx + part - 1) / part;
  if (np > 65535 * 32) return fail(PA_ERR_ARG, "partition_size too small for this table width");

  pa::DecodeArgs a;
  std::memset(&a, 0, sizeof a);
  a.out = out.data;
  a.q = q.data;
  a.k_cache = k_cache.data;
  a.v_cache = v_cache.data;
  a.block_tables = static_cast<const int32_t *>(block_tables.data);
  a.context_lens = static_cast<const int32_t *>(context_lens.data);
  if (np > 1) {
    const size_t need = pa_decode_workspace_size(S, H, num_kv_heads, D, W, block_size, (int32_t)part);
    if (!o.workspace || o.workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  o.workspace ? o.workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(o.workspace) % 16) return fail(PA_ERR_LAYOUT, "workspace not 16-byte aligned");
    const int64_t rows = S * H * np;
    a.ws_ml = static_cast<float *>(o.workspace);
    a.ws_acc = a.ws_ml + rows * 2;
  }
  a.q_ss = q.stride[0];
  a.q_sh = q.stride[1];
  a.o_ss = out.stride[0];
  a.o_sh = out.stride[1];
  a.k_sb = k_cache.stride[0];
  a.k_st = k_cache.stride[1];
  a.k_sh = k_cache.stride[2];
  a.v_sb = v_cache.stride[0];
  a.v_st = v_cache.stride[1];
  a.v_sh = v_cache.stride[2];
  a.bt_ss = block_tables.stride[0];
  a.num_seqs = (int32_t)S;
  a.num_heads = (int32_t)H;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = (int32_t)D;
  a.num_blocks = (int32_t)NB;
  a.block_size = block_size;
  a.log2_block_size = block_size == 16 ? 4 : 5;
  a.max_blocks_per_seq = (int32_t)W;
  a.max_ctx = (int32_t)max_ctx;
  a.partition_size = (int32_t)part;
  a.num_partitions = (int32_t)np;
  a.qk_scale_log2 = (float)((double)scale * 1.4426950408889634 * (double)ks);
  a.v_scale = vs;
  a.kv_kind = kvk;
  a.q_kind = kv_kind(q.dtype);
  a.out_f32 = out.dtype == PA_F32 && q.dtype != PA_F32;

  hipStream_t stream = static_cast<hipStream_t>(o.stream);
  hipError_t e = pa::launch_decode_partitions(a, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "partition kernel launch: %s", hipGetErrorString(e));
  if (o.mark_event) {
    e = hipEventRecord(static_cast<hipEvent_t>(o.mark_event), stream);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  }
  if (np > 1) {
    e = pa::launch_decode_reduce(a, stream);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "reduce kernel launch: %s", hipGetErrorString(e));
  }
  return PA_OK;
}

pa_status pa_cache_write(pa_tensor k, pa_tensor v, pa_tensor k_cache, pa_tensor v_cache, pa_tensor slot_mapping,
                         const pa_opts *opts) {
  pa_opts o;
  std::memset(&o, 0, sizeof o);
  if (opts) o = *opts;
  pa_status st;
  if ((st = check_tensor(k, "k", 3, true))) return st;
  if ((st = check_tensor(v, "v", 3, true))) return st;
  if ((st = check_tensor(k_cache, "k_cache", 4, true))) return st;
  if ((st = check_tensor(v_cache, "v_cache", 4, true))) return st;
  if ((st = check_tensor(slot_mapping, "slot_mapping", 1, false))) return st;
  if (slot_mapping.dtype != PA_I64 && slot_mapping.dtype != PA_I32)
    return fail(PA_ERR_DTYPE, "slot_mapping: dtype must be I64 or I32");
  if (k.dtype != v.dtype) return fail(PA_ERR_DTYPE, "k and v dtypes differ");
  if (k_cache.dtype != v_cache.dtype) return fail(PA_ERR_DTYPE, "k_cache and v_cache dtypes differ");
  const int ck = kv_kind(k_cache.dtype), ik = kv_kind(k.dtype);
  if (ck < 0 || ik < 0) return fail(PA_ERR_DTYPE, "k and caches must be F32, F16, BF16 or FP8_E4M3");
  if (ik != ck && ck != pa::KV_FP8) return fail(PA_ERR_DTYPE, "k dtype must equal the cache dtype");
  for (int i = 0; i < 3; ++i)
    if (k.shape[i] != v.shape[i]) return fail(PA_ERR_SHAPE, "k and v shapes differ");
  for (int i = 0; i < 4; ++i)
    if (k_cache.shape[i] != v_cache.shape[i]) return fail(PA_ERR_SHAPE, "k_cache and v_cache shapes differ");
  const int64_t N = k.shape[0], Hkv = k.shape[1], D = k.shape[2];
  if (k_cache.shape[2] != Hkv || k_cache.shape[3] != D)
    return fail(PA_ERR_SHAPE, "k is [%lld, %lld, %lld], cache rows are [%lld, %lld]", (long long)N, (long long)Hkv,
                (long long)D, (long long)k_cache.shape[2], (long long)k_cache.shape[3]);
  if (slot_mapping.shape[0] != N) return fail(PA_ERR_SHAPE, "slot_mapping has %lld entries, k has %lld tokens",
                                              (long long)slot_mapping.shape[0], (long long)N);
  const int64_t vec = ck == pa::KV_FP8 ? 16 : 16 / elem_bytes(k_cache.dtype);
  if (D % vec) return fail(PA_ERR_UNSUPPORTED, "head_dim %lld not a multiple of %lld", (long long)D, (long long)vec);
  if (N > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "too many tokens");
  float ks = o.k_scale == 0.0f ? 1.0f : o.k_scale, vs = o.v_scale == 0.0f ? 1.0f : o.v_scale;
  if (!(ks > 0.0f) || !std::isfinite(ks) || !(vs > 0.0f) || !std::isfinite(vs))
    return fail(PA_ERR_ARG, "k_scale / v_scale must be finite and > 0");
  if (o.flags != 0) return fail(PA_ERR_ARG, "flags must be 0");
  if (N == 0 || Hkv == 0 || D == 0) return PA_OK;

  pa::CacheWriteArgs a;
  std::memset(&a, 0, sizeof a);
  a.k = k.data;
  a.v = v.data;
  a.k_cache = k_cache.data;
  a.v_cache = v_cache.data;
  a.slot_mapping = slot_mapping.data;
  a.slot_i64 = slot_mapping.dtype == PA_I64;
  a.k_sn = k.stride[0];
  a.k_sh = k.stride[1];
  a.v_sn = v.stride[0];
  a.v_sh = v.stride[1];
  a.kc_sb = k_cache.stride[0];
  a.kc_st = k_cache.stride[1];
  a.kc_sh = k_cache.stride[2];
  a.vc_sb = v_cache.stride[0];
  a.vc_st = v_cache.stride[1];
  a.vc_sh = v_cache.stride[2];
  a.num_tokens = (int32_t)N;
  a.num_kv_heads = (int32_t)Hkv;
  a.head_dim = (int32_t)D;
  a.num_slots = k_cache.shape[0] * k_cache.shape[1];
  a.block_size = (int32_t)k_cache.shape[1];
  a.in_kind = ik;
  a.cache_kind = ck;
  a.k_scale = ks;
  a.v_scale = vs;
  if (a.block_size <= 0) return fail(PA_ERR_SHAPE, "block_size must be positive");
  hipError_t e = pa::launch_cache_write(a, static_cast<hipStream_t>(o.stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "cache-write kernel launch: %s", hipGetErrorString(e));
  return PA_OK;
}

const char *pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer";
    case PA_ERR_DTYPE: return "unsupported dtype";
    case PA_ERR_SHAPE: return "shape mismatch";
    case PA_ERR_LAYOUT: return "unsupported layout or alignment";
    case PA_ERR_UNSUPPORTED: return "configuration not built";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_ARG: return "argument out of range";
    case PA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *pa_last_error(void) { return g_last_error; }

const char *pa_version(void) { return "0.1.0"; }

}  // extern "C"
