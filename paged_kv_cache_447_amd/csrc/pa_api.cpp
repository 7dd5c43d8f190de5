// Host side of the C ABI declared in include/pa.h: argument validation, the
// work-split choice, workspace carving and kernel dispatch.  Nothing here
// allocates device memory or waits for the device.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "pa_internal.h"
#include "pa_validate.h"

namespace {

thread_local char g_last_error[512] = "";

pa_status fail(pa_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

}  // namespace

namespace pa {
pa_status fail_message(pa_status s, const char *msg) { return fail(s, "%s", msg); }
}  // namespace pa

namespace {

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

// rank, non-null data, non-negative strides, contiguous last dimension,
// 16-byte alignment of the base and of every outer stride (vector loads/stores
// address whole rows) (an empty tensor may have a NULL data pointer)
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
  for (int i = 0; i < ndim; ++i)
    if (t.stride[i] < 0 && t.shape[i] > 1) return fail(PA_ERR_LAYOUT, "%s: negative stride in dim %d", name, i);
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

// The attention kernels address a row inside a block by a 32-bit byte offset
// from the block's start: (block_size - 1) token strides plus one row must stay
// below 4 GiB (a token-major view of a very large pool can exceed that).
pa_status check_block_extent(const pa_tensor &c, const char *name) {
  const int64_t eb = elem_bytes(c.dtype), st = c.stride[1];
  if (c.shape[0] == 0 || c.shape[1] == 0) return PA_OK;
  if (st >= ((int64_t)1 << 32) || ((c.shape[1] - 1) * st + c.shape[3]) * eb >= ((int64_t)1 << 32))
    return fail(PA_ERR_LAYOUT, "%s: a block spans 4 GiB or more (token stride %lld elements)", name, (long long)st);
  return PA_OK;
}

// opts->flags: PA_FLAG_VALIDATE or nothing
pa_status check_flags(const pa_opts &o) {
  if ((o.flags & ~PA_FLAG_VALIDATE) != 0 || o.reserved != 0)
    return fail(PA_ERR_ARG, "flags: only PA_FLAG_VALIDATE is defined; reserved must be 0");
  return PA_OK;
}

constexpr int kWavesPerWG = 4;
constexpr int64_t kMaxWorkers = 1 << 20;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Workers per compute unit when the caller leaves the choice to the library:
// one wavefront per SIMD.  Each keeps a chunk of K or V in flight; more
// workers only add segment starts and partials to merge.
constexpr int kDefaultWorkersPerCU = 4;

int32_t device_default_workers() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  // a multiple of 8 workgroups, so that every XCD gets the same number
  return (int32_t)round_up((int64_t)cus * kDefaultWorkersPerCU, 8 * kWavesPerWG);
}

int32_t effective_workers(int32_t requested) {
  if (requested <= 0) return device_default_workers();
  int64_t w = round_up(requested, kWavesPerWG);
  return (int32_t)(w > kMaxWorkers ? kMaxWorkers : w);
}

// The decode workspace: the partial-result slots from its start (the (max,
// sum) pairs, then the outputs), the merge counters at its end.  A call
// leaves its counters at zero and garbage in its slots; the slots' extent
// depends only on the group size, head_dim and worker count, and the counters
// sit past it whatever the batch, so calls with those three in common may
// share a workspace whatever their number of sequences or layers: each
// call's counters lie where earlier calls left zeros.
struct WsLayout {
  size_t ml, acc, parts;  // byte offsets of the two slot regions, and where the slots end
  size_t counters_bytes;  // the counters' region (at the end of the workspace)
  size_t total;           // bytes needed
  // the counters' offset in a workspace of `bytes` (>= total) bytes
  size_t counters(size_t bytes) const { return bytes / 256 * 256 - counters_bytes; }
};

WsLayout workspace_layout(int64_t S, int64_t H, int64_t Hkv, int64_t D, int64_t W) {
  WsLayout l;
  const int64_t G = H / Hkv;
  const int64_t slots = 2 * W;
  l.ml = 0;
  l.acc = (size_t)round_up(slots * G * 2 * 4, 256);
  l.parts = l.acc + (size_t)round_up(slots * G * D * 4, 256);
  l.counters_bytes = (size_t)round_up(S * Hkv * 4, 256);
  l.total = l.parts + l.counters_bytes;
  return l;
}

// The device address of memory the GPU can reach: device memory, or pinned
// host memory mapped into the device's address space.  Pageable host memory
// (or anything unknown to the runtime) is refused, so a kernel never touches it.
pa_status device_address(const void *p, const char *name, void **dev) {
  hipPointerAttribute_t at;
  std::memset(&at, 0, sizeof at);
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PA_ERR_ARG, "%s: not device memory or pinned host memory", name);
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) {
    *dev = const_cast<void *>(p);
    return PA_OK;
  }
  if (at.type == hipMemoryTypeHost && at.devicePointer) {
    // the mapped alias of this byte (the attributes describe the allocation's base)
    const char *hbase = static_cast<const char *>(at.hostPointer ? at.hostPointer : p);
    *dev = static_cast<char *>(at.devicePointer) + (static_cast<const char *>(p) - hbase);
    return PA_OK;
  }
  return fail(PA_ERR_ARG, "%s: not device memory or pinned host memory", name);
}

// The argument checks of per-kv-head fp8 scales that need no device: both or
// neither, fp8 caches only.
pa_status check_head_scale_args(const pa_opts &o, int cache_kind) {
  if (!o.k_head_scales && !o.v_head_scales) return PA_OK;
  if (!o.k_head_scales || !o.v_head_scales) return fail(PA_ERR_NULL, "k_head_scales and v_head_scales go together");
  if (cache_kind != pa::KV_FP8) return fail(PA_ERR_ARG, "per-head scales apply to FP8_E4M3 caches only");
  return PA_OK;
}

// Per-kv-head fp8 scales of opts (as above, and not together with per-tensor
// scales), as device addresses; null when not given.
pa_status head_scales(const pa_opts &o, int cache_kind, const float **ks, const float **vs) {
  *ks = *vs = nullptr;
  pa_status st;
  if ((st = check_head_scale_args(o, cache_kind))) return st;
  if (!o.k_head_scales) return PA_OK;
  if (o.k_scale != 0.0f || o.v_scale != 0.0f)
    return fail(PA_ERR_ARG, "per-tensor and per-head scales exclude each other: leave k_scale and v_scale at 0");
  if (reinterpret_cast<uintptr_t>(o.k_head_scales) % 4 || reinterpret_cast<uintptr_t>(o.v_head_scales) % 4)
    return fail(PA_ERR_LAYOUT, "per-head scales must be 4-byte aligned");
  void *dk = nullptr, *dv = nullptr;
  if ((st = device_address(o.k_head_scales, "k_head_scales", &dk))) return st;
  if ((st = device_address(o.v_head_scales, "v_head_scales", &dv))) return st;
  *ks = static_cast<const float *>(dk);
  *vs = static_cast<const float *>(dv);
  return PA_OK;
}

// Per-(block, kv head) fp8 scales of opts: both or neither, fp8 caches only,
// not with per-head or per-tensor scales; device addresses, or null when not given.
pa_status block_scales(const pa_opts &o, int cache_kind, const float **kb, const float **vb) {
  *kb = *vb = nullptr;
  if (!o.k_block_scales && !o.v_block_scales) return PA_OK;
  if (!o.k_block_scales || !o.v_block_scales) return fail(PA_ERR_NULL, "k_block_scales and v_block_scales go together");
  if (cache_kind != pa::KV_FP8) return fail(PA_ERR_ARG, "per-block scales apply to FP8_E4M3 caches only");
  if (o.k_head_scales || o.v_head_scales) return fail(PA_ERR_ARG, "per-block and per-head scales exclude each other");
  if (o.k_scale != 0.0f || o.v_scale != 0.0f)
    return fail(PA_ERR_ARG, "per-tensor and per-block scales exclude each other: leave k_scale and v_scale at 0");
  if (reinterpret_cast<uintptr_t>(o.k_block_scales) % 4 || reinterpret_cast<uintptr_t>(o.v_block_scales) % 4)
    return fail(PA_ERR_LAYOUT, "per-block scales must be 4-byte aligned");
  void *dk = nullptr, *dv = nullptr;
  pa_status st;
  if ((st = device_address(o.k_block_scales, "k_block_scales", &dk))) return st;
  if ((st = device_address(o.v_block_scales, "v_block_scales", &dv))) return st;
  *kb = static_cast<const float *>(dk);
  *vb = static_cast<const float *>(dv);
  return PA_OK;
}

}  // namespace

extern "C" {

int32_t pa_decode_num_workers(int32_t requested) { return effective_workers(requested); }

size_t pa_prefill_workspace_size(void) { return 256; }

size_t pa_decode_workspace_size(int64_t num_seqs, int64_t num_heads, int64_t num_kv_heads, int64_t head_dim,
                                int32_t num_workers) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_heads % num_kv_heads) return 0;
  return workspace_layout(num_seqs, num_heads, num_kv_heads, head_dim, effective_workers(num_workers)).total;
}

}  // extern "C"

namespace {

// The new tokens of pa_decode_append.
struct AppendIn {
  pa_tensor k_new, v_new, slot_mapping;
};

// pa_decode over one layer (layers = 1, strides 0), or over several layers
// whose per-layer views out/q/k_cache/v_cache are given with the layer
// strides (elements) between consecutive layers; with `ap`, the one-layer
// step that also stores every sequence's new token (pa_decode_append).
pa_status decode_impl(pa_tensor out, pa_tensor q, pa_tensor k_cache, pa_tensor v_cache, pa_tensor block_tables,
                      pa_tensor context_lens, int32_t block_size, float scale, int32_t num_kv_heads,
                      const pa_opts *opts, int64_t layers, int64_t q_sl, int64_t o_sl, int64_t k_sl, int64_t v_sl,
                      const AppendIn *ap = nullptr) {
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
                "(built: head_dim 64/128, group 1/2/4/8, 16 for 16-bit or fp8 caches)", (long long)D, (long long)(H / num_kv_heads));
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(PA_ERR_ARG, "scale must be finite and > 0");
  float ks = o.k_scale == 0.0f ? 1.0f : o.k_scale, vs = o.v_scale == 0.0f ? 1.0f : o.v_scale;
  if (kvk != pa::KV_FP8) ks = vs = 1.0f;
  if (!(ks > 0.0f) || !std::isfinite(ks) || !(vs > 0.0f) || !std::isfinite(vs))
    return fail(PA_ERR_ARG, "k_scale / v_scale must be finite and > 0");
  if ((st = check_flags(o))) return st;
  if ((st = check_head_scale_args(o, kvk))) return st;
  if ((st = check_block_extent(k_cache, "k_cache"))) return st;
  if ((st = check_block_extent(v_cache, "v_cache"))) return st;
  const int64_t W = block_tables.shape[1];
  if (S > 65535 || num_kv_heads > 65535) return fail(PA_ERR_UNSUPPORTED, "more than 65535 sequences or kv heads");
  if (W * block_size > (int64_t)1 << 30) return fail(PA_ERR_UNSUPPORTED, "table width too large");
  if (NB > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "more than 2^31-1 blocks");
  if (S == 0 || H == 0) return PA_OK;
  if (NB == 0 || W == 0) return fail(PA_ERR_SHAPE, "empty cache or block table");

  if (layers < 1 || S * layers > 65535) return fail(PA_ERR_UNSUPPORTED, "more than 65535 (layer, sequence) pairs");
  const int G = (int)(H / num_kv_heads);
  const int64_t max_ctx = W * block_size;
  int64_t part = o.partition_size;
  if (part == 0) part = pa::decode_chunk_tokens(kvk, (int)D, G);
  if (part <= 0 || (o.partition_size && part % block_size))
    return fail(PA_ERR_ARG, "partition_size %lld must be a positive multiple of block_size", (long long)part);
  if ((max_ctx + part - 1) / part > ((int64_t)1 << 24))
    return fail(PA_ERR_ARG, "partition_size %lld too small for a table of %lld tokens", (long long)part,
                (long long)max_ctx);
  if (o.num_workers < 0) return fail(PA_ERR_ARG, "num_workers must be >= 0");
  if (layers * S * num_kv_heads * ((max_ctx + part - 1) / part) > ((int64_t)1 << 40))
    return fail(PA_ERR_UNSUPPORTED, "too many work units");
  const int32_t nw = effective_workers(o.num_workers);
  const WsLayout ws = workspace_layout(layers * S, H, num_kv_heads, D, nw);
  if (ws.parts - ws.acc >= ((size_t)1 << 32))  // partial slots are addressed with 32-bit byte offsets
    return fail(PA_ERR_UNSUPPORTED, "num_workers %d too large for this head shape", nw);
  if (!o.workspace || o.workspace_bytes < ws.total)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws.total,
                o.workspace ? o.workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(o.workspace) % 256) return fail(PA_ERR_WORKSPACE, "workspace not 256-byte aligned");

  const float *khs = nullptr, *vhs = nullptr, *kbs = nullptr, *vbs = nullptr;
  if ((st = head_scales(o, kvk, &khs, &vhs))) return st;
  if ((st = block_scales(o, kvk, &kbs, &vbs))) return st;
  if (ap) {
    if ((st = check_tensor(ap->k_new, "k_new", 3, true))) return st;
    if ((st = check_tensor(ap->v_new, "v_new", 3, true))) return st;
    if ((st = check_tensor(ap->slot_mapping, "slot_mapping", 1, false))) return st;
    if (kvk == pa::KV_FP8)
      return fail(PA_ERR_UNSUPPORTED, "fp8 caches: write the new tokens with pa_cache_write, then pa_decode");
    if (ap->k_new.dtype != k_cache.dtype || ap->v_new.dtype != k_cache.dtype)
      return fail(PA_ERR_DTYPE, "k_new and v_new must have the caches' dtype");
    if (ap->slot_mapping.dtype != PA_I64 && ap->slot_mapping.dtype != PA_I32)
      return fail(PA_ERR_DTYPE, "slot_mapping: dtype must be I64 or I32");
    for (const pa_tensor *t : {&ap->k_new, &ap->v_new})
      if (t->shape[0] != S || t->shape[1] != num_kv_heads || t->shape[2] != D)
        return fail(PA_ERR_SHAPE, "k_new and v_new must be [num_seqs, num_kv_heads, head_dim]");
    if (ap->slot_mapping.shape[0] != S) return fail(PA_ERR_SHAPE, "slot_mapping must have one entry per sequence");
    if (layers != 1) return fail(PA_ERR_UNSUPPORTED, "the fused step takes one layer");
  }
  if (o.flags & PA_FLAG_VALIDATE) {
    const hipStream_t stream = static_cast<hipStream_t>(o.stream);
    pa::HostInts bt, lens, slots;
    if ((st = pa::validation_allowed(stream))) return st;
    if ((st = bt.fetch(block_tables, "block_tables", stream))) return st;
    if ((st = lens.fetch(context_lens, "context_lens", stream))) return st;
    if ((st = pa::check_tables(bt, lens, block_size, NB))) return st;
    if (ap) {
      if ((st = slots.fetch(ap->slot_mapping, "slot_mapping", stream))) return st;
      if ((st = pa::check_new_token_slots(slots, bt, lens, block_size, NB * block_size))) return st;
    }
    if ((st = pa::check_head_scales(khs, vhs, layers * num_kv_heads, stream))) return st;
    if ((st = pa::check_head_scales(kbs, vbs, layers * NB * num_kv_heads, stream, "k_block_scales", "v_block_scales")))
      return st;
  }

  pa::DecodeArgs a;
  std::memset(&a, 0, sizeof a);
  a.out = out.data;
  a.q = q.data;
  a.k_cache = k_cache.data;
  a.v_cache = v_cache.data;
  a.block_tables = static_cast<const int32_t *>(block_tables.data);
  a.context_lens = static_cast<const int32_t *>(context_lens.data);
  char *wsb = static_cast<char *>(o.workspace);
  a.counters = reinterpret_cast<int32_t *>(wsb + ws.counters(o.workspace_bytes));
  a.part_ml = reinterpret_cast<float *>(wsb + ws.ml);
  a.part_acc = reinterpret_cast<float *>(wsb + ws.acc);
  a.ml_bytes = (uint32_t)(ws.acc - ws.ml);
  a.acc_bytes = (uint32_t)(ws.parts - ws.acc);
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
  a.num_seqs = (int32_t)(S * layers);
  a.seqs_per_layer = (int32_t)S;
  a.q_sl = q_sl;
  a.o_sl = o_sl;
  a.k_sl = k_sl;
  a.v_sl = v_sl;
  a.num_heads = (int32_t)H;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = (int32_t)D;
  a.num_blocks = (int32_t)NB;
  a.block_size = block_size;
  a.max_blocks_per_seq = (int32_t)W;
  a.max_ctx = (int32_t)max_ctx;
  a.part_tokens = (int32_t)part;
  a.num_workers = nw;
  a.qk_scale_log2 = (float)((double)scale * 1.4426950408889634 * (double)ks);
  a.v_scale = vs;
  a.k_head_scale = khs;
  a.v_head_scale = vhs;
  a.k_block_scale = kbs;
  a.v_block_scale = vbs;
  a.kv_kind = kvk;
  a.q_kind = kv_kind(q.dtype);
  a.out_f32 = out.dtype == PA_F32 && q.dtype != PA_F32;
  if (ap) {
    a.append = 1;
    a.k_new = ap->k_new.data;
    a.v_new = ap->v_new.data;
    a.kn_ss = ap->k_new.stride[0];
    a.kn_sh = ap->k_new.stride[1];
    a.vn_ss = ap->v_new.stride[0];
    a.vn_sh = ap->v_new.stride[1];
    a.slot_mapping = ap->slot_mapping.data;
    a.slot_i64 = ap->slot_mapping.dtype == PA_I64;
    a.num_slots = NB * block_size;
  }

  hipError_t e = pa::launch_decode(a, static_cast<hipStream_t>(o.stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "decode kernel launch: %s", hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

namespace pa {
// Bytes at the start of a decode workspace that a call with this head shape
// and worker request may leave non-zero (its partial-result slots).
size_t decode_partials_bytes(int64_t num_heads, int64_t num_kv_heads, int64_t head_dim, int32_t num_workers) {
  if (num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_heads % num_kv_heads) return 0;
  return workspace_layout(1, num_heads, num_kv_heads, head_dim, effective_workers(num_workers)).parts;
}

// pa_decode on a workspace the library provides (opts->workspace must be
// NULL): the entry point for callers that cannot allocate.
pa_status decode_with_workspace(pa_tensor out, pa_tensor q, pa_tensor k_cache, pa_tensor v_cache,
                                pa_tensor block_tables, pa_tensor context_lens, int32_t block_size, float scale,
                                int32_t num_kv_heads, const pa_opts *opts, void *workspace, size_t workspace_bytes) {
  pa_opts o;
  std::memset(&o, 0, sizeof o);
  if (opts) o = *opts;
  if (o.workspace || o.workspace_bytes)
    return fail(PA_ERR_ARG, "opts->workspace must be NULL: this entry point uses the library's own scratch");
  o.workspace = workspace;
  o.workspace_bytes = workspace_bytes;
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, block_size, scale, num_kv_heads, &o, 1, 0,
                     0, 0, 0);
}
}  // namespace pa

namespace {

// The view of one layer of a [layers, ...] tensor: the leading dimension dropped.
pa_tensor layer_view(const pa_tensor &t) {
  pa_tensor v;
  std::memset(&v, 0, sizeof v);
  v.data = t.data;
  v.dtype = t.dtype;
  v.ndim = t.ndim - 1;
  for (int i = 1; i < t.ndim; ++i) {
    v.shape[i - 1] = t.shape[i];
    v.stride[i - 1] = t.stride[i];
  }
  return v;
}

}  // namespace

extern "C" {

pa_status pa_decode(pa_tensor out, pa_tensor q, pa_tensor k_cache, pa_tensor v_cache, pa_tensor block_tables,
                    pa_tensor context_lens, int32_t block_size, float scale, int32_t num_kv_heads,
                    const pa_opts *opts) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, block_size, scale, num_kv_heads, opts, 1,
                     0, 0, 0, 0);
}

pa_status pa_decode_append(pa_tensor out, pa_tensor q, pa_tensor k_new, pa_tensor v_new, pa_tensor k_cache,
                           pa_tensor v_cache, pa_tensor slot_mapping, pa_tensor block_tables, pa_tensor context_lens,
                           int32_t block_size, float scale, int32_t num_kv_heads, const pa_opts *opts) {
  const AppendIn ap{k_new, v_new, slot_mapping};
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, block_size, scale, num_kv_heads, opts, 1,
                     0, 0, 0, 0, &ap);
}

pa_status pa_decode_layers(pa_tensor out, pa_tensor q, pa_tensor k_caches, pa_tensor v_caches,
                           pa_tensor block_tables, pa_tensor context_lens, int32_t block_size, float scale,
                           int32_t num_kv_heads, const pa_opts *opts) {
  if (out.ndim != 4 || q.ndim != 4) return fail(PA_ERR_SHAPE, "out and q must be [layers, num_seqs, num_heads, head_dim]");
  if (k_caches.ndim != 5 || v_caches.ndim != 5)
    return fail(PA_ERR_SHAPE, "caches must be [layers, num_blocks, block_size, num_kv_heads, head_dim]");
  const int64_t L = q.shape[0];
  if (out.shape[0] != L || k_caches.shape[0] != L || v_caches.shape[0] != L)
    return fail(PA_ERR_SHAPE, "out, q, k_caches and v_caches must have the same number of layers");
  if (L < 0) return fail(PA_ERR_SHAPE, "negative layer count");
  if (L == 0) return PA_OK;
  const pa_tensor *ts[4] = {&out, &q, &k_caches, &v_caches};
  for (const pa_tensor *t : ts) {
    const int eb = elem_bytes(t->dtype);
    if (eb && L > 1 && (t->stride[0] * eb) % 16) return fail(PA_ERR_LAYOUT, "layer stride not a multiple of 16 bytes");
  }
  return decode_impl(layer_view(out), layer_view(q), layer_view(k_caches), layer_view(v_caches), block_tables,
                     context_lens, block_size, scale, num_kv_heads, opts, L, q.stride[0], out.stride[0],
                     k_caches.stride[0], v_caches.stride[0]);
}

pa_status pa_prefill(pa_tensor out, pa_tensor q, pa_tensor k_cache, pa_tensor v_cache, pa_tensor block_tables,
                     pa_tensor context_lens, pa_tensor query_start_loc, int32_t block_size, float scale,
                     int32_t num_kv_heads, const pa_opts *opts) {
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
  if ((st = check_tensor(query_start_loc, "query_start_loc", 1, false))) return st;

  if (q.dtype != PA_F16 && q.dtype != PA_BF16) return fail(PA_ERR_DTYPE, "q: dtype must be F16 or BF16");
  if (k_cache.dtype != v_cache.dtype) return fail(PA_ERR_DTYPE, "k_cache and v_cache dtypes differ");
  if (k_cache.dtype != q.dtype && k_cache.dtype != PA_FP8_E4M3)
    return fail(PA_ERR_DTYPE, "k_cache and v_cache must have q's dtype or FP8_E4M3");
  if (out.dtype != q.dtype && out.dtype != PA_F32) return fail(PA_ERR_DTYPE, "out: dtype must be q's dtype or F32");
  if (block_tables.dtype != PA_I32) return fail(PA_ERR_DTYPE, "block_tables: dtype must be I32");
  if (context_lens.dtype != PA_I32) return fail(PA_ERR_DTYPE, "context_lens: dtype must be I32");
  if (query_start_loc.dtype != PA_I32) return fail(PA_ERR_DTYPE, "query_start_loc: dtype must be I32");

  const int64_t N = q.shape[0], H = q.shape[1], D = q.shape[2];
  const int64_t S = context_lens.shape[0], NB = k_cache.shape[0];
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
  if (num_kv_heads <= 0 || H % num_kv_heads)
    return fail(PA_ERR_SHAPE, "num_heads %lld not a multiple of num_kv_heads %d", (long long)H, num_kv_heads);
  if (block_tables.shape[0] != S) return fail(PA_ERR_SHAPE, "block_tables has %lld rows, context_lens %lld entries",
                                              (long long)block_tables.shape[0], (long long)S);
  if (query_start_loc.shape[0] != S + 1)
    return fail(PA_ERR_SHAPE, "query_start_loc has %lld entries, expected num_seqs + 1 = %lld",
                (long long)query_start_loc.shape[0], (long long)(S + 1));
  if (block_size != 16 && block_size != 32) return fail(PA_ERR_UNSUPPORTED, "block_size %d (built: 16, 32)", block_size);
  if (!pa::prefill_supported(kv_kind(k_cache.dtype), (int)D))
    return fail(PA_ERR_UNSUPPORTED, "no prefill kernel for head_dim %lld (built: 64, 128)", (long long)D);
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(PA_ERR_ARG, "scale must be finite and > 0");
  if ((st = check_flags(o))) return st;
  if ((st = check_head_scale_args(o, kv_kind(k_cache.dtype)))) return st;
  if ((st = check_block_extent(k_cache, "k_cache"))) return st;
  if ((st = check_block_extent(v_cache, "v_cache"))) return st;
  float ks = o.k_scale == 0.0f ? 1.0f : o.k_scale, vs = o.v_scale == 0.0f ? 1.0f : o.v_scale;
  if (k_cache.dtype != PA_FP8_E4M3) ks = vs = 1.0f;
  if (!(ks > 0.0f) || !std::isfinite(ks) || !(vs > 0.0f) || !std::isfinite(vs))
    return fail(PA_ERR_ARG, "k_scale / v_scale must be finite and > 0");
  const int64_t W = block_tables.shape[1];
  const int64_t G = num_kv_heads > 0 ? H / num_kv_heads : 0;
  if (S > INT32_MAX - 1 || N * G > INT32_MAX / 2) return fail(PA_ERR_UNSUPPORTED, "too many sequences or query rows");
  if (W * block_size > (int64_t)1 << 30) return fail(PA_ERR_UNSUPPORTED, "table width too large");
  if (NB > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "more than 2^31-1 blocks");
  if (S == 0 || N == 0 || H == 0) return PA_OK;
  if (NB == 0 || W == 0) return fail(PA_ERR_SHAPE, "empty cache or block table");

  pa::PrefillArgs a;
  std::memset(&a, 0, sizeof a);
  a.out = out.data;
  a.q = q.data;
  a.k_cache = k_cache.data;
  a.v_cache = v_cache.data;
  a.block_tables = static_cast<const int32_t *>(block_tables.data);
  a.context_lens = static_cast<const int32_t *>(context_lens.data);
  a.query_start_loc = static_cast<const int32_t *>(query_start_loc.data);
  a.q_sn = q.stride[0];
  a.q_sh = q.stride[1];
  a.o_sn = out.stride[0];
  a.o_sh = out.stride[1];
  a.k_sb = k_cache.stride[0];
  a.k_st = k_cache.stride[1];
  a.k_sh = k_cache.stride[2];
  a.v_sb = v_cache.stride[0];
  a.v_st = v_cache.stride[1];
  a.v_sh = v_cache.stride[2];
  a.bt_ss = block_tables.stride[0];
  a.num_seqs = (int32_t)S;
  a.num_rows = (int32_t)N;
  a.num_heads = (int32_t)H;
  a.num_kv_heads = num_kv_heads;
  a.group = (int32_t)G;
  a.head_dim = (int32_t)D;
  a.num_blocks = (int32_t)NB;
  a.block_size = block_size;
  a.max_ctx = (int32_t)(W * block_size);
  int tile_cols = 0, key_split = 0;
  pa::prefill_plan(N, S, (int)G, tile_cols, key_split);
  a.tile_cols = tile_cols;
  a.key_split = key_split;
  a.persistent_wgs = device_default_workers() / kDefaultWorkersPerCU;  // one workgroup per CU
  // every sequence's tiles: at most N * G / tile_cols whole ones plus one partial tile each
  const int64_t slots = (N * G + a.tile_cols - 1) / a.tile_cols + S;
  if (slots * num_kv_heads > INT32_MAX / 2) return fail(PA_ERR_UNSUPPORTED, "too many tiles");
  a.tile_slots = (int32_t)slots;
  if ((st = head_scales(o, kv_kind(k_cache.dtype), &a.k_head_scale, &a.v_head_scale))) return st;
  if ((st = block_scales(o, kv_kind(k_cache.dtype), &a.k_block_scale, &a.v_block_scale))) return st;
  if (o.workspace) {  // the key split's pair counter
    if (o.workspace_bytes < pa_prefill_workspace_size())
      return fail(PA_ERR_WORKSPACE, "prefill workspace of %zu bytes needed, %zu given", pa_prefill_workspace_size(),
                  o.workspace_bytes);
    if (reinterpret_cast<uintptr_t>(o.workspace) % 256) return fail(PA_ERR_WORKSPACE, "workspace not 256-byte aligned");
    a.pair_counter = static_cast<int32_t *>(o.workspace);
  }
  if (o.flags & PA_FLAG_VALIDATE) {
    const hipStream_t stream = static_cast<hipStream_t>(o.stream);
    pa::HostInts bt, lens, qsl;
    if ((st = pa::validation_allowed(stream))) return st;
    if ((st = bt.fetch(block_tables, "block_tables", stream))) return st;
    if ((st = lens.fetch(context_lens, "context_lens", stream))) return st;
    if ((st = qsl.fetch(query_start_loc, "query_start_loc", stream))) return st;
    if ((st = pa::check_tables(bt, lens, block_size, NB))) return st;
    if ((st = pa::check_query_starts(qsl, lens, N))) return st;
    if ((st = pa::check_head_scales(a.k_head_scale, a.v_head_scale, num_kv_heads, stream))) return st;
    if ((st = pa::check_head_scales(a.k_block_scale, a.v_block_scale, NB * num_kv_heads, stream, "k_block_scales",
                                    "v_block_scales")))
      return st;
  }
  a.qk_scale_log2 = (float)((double)scale * 1.4426950408889634 * (double)ks);
  a.v_scale = vs;
  a.kv_kind = kv_kind(k_cache.dtype);
  a.q_kind = kv_kind(q.dtype);
  a.out_f32 = out.dtype == PA_F32;

  hipError_t e = pa::launch_prefill(a, static_cast<hipStream_t>(o.stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "prefill kernel launch: %s", hipGetErrorString(e));
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
  if ((st = check_flags(o))) return st;
  if ((st = check_head_scale_args(o, ck))) return st;
  if (N == 0 || Hkv == 0 || D == 0) return PA_OK;
  const float *khs = nullptr, *vhs = nullptr, *kbs = nullptr, *vbs = nullptr;
  if ((st = head_scales(o, ck, &khs, &vhs))) return st;
  if ((st = block_scales(o, ck, &kbs, &vbs))) return st;
  if (o.flags & PA_FLAG_VALIDATE) {
    const hipStream_t stream = static_cast<hipStream_t>(o.stream);
    pa::HostInts slots;
    if ((st = pa::validation_allowed(stream))) return st;
    if ((st = slots.fetch(slot_mapping, "slot_mapping", stream))) return st;
    if ((st = pa::check_distinct_slots(slots, k_cache.shape[0] * k_cache.shape[1]))) return st;
    if (ik != pa::KV_FP8 && (st = pa::check_head_scales(khs, vhs, Hkv, stream))) return st;
    if ((st = pa::check_head_scales(kbs, vbs, k_cache.shape[0] * Hkv, stream, "k_block_scales", "v_block_scales")))
      return st;
  }

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
  a.k_head_scale = khs;
  a.v_head_scale = vhs;
  a.k_block_scale = kbs;
  a.v_block_scale = vbs;
  if (a.block_size <= 0) return fail(PA_ERR_SHAPE, "block_size must be positive");
  hipError_t e = pa::launch_cache_write(a, static_cast<hipStream_t>(o.stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "cache-write kernel launch: %s", hipGetErrorString(e));
  return PA_OK;
}

pa_status pa_copy_blocks(pa_tensor dst_k_cache, pa_tensor dst_v_cache, pa_tensor src_k_cache, pa_tensor src_v_cache,
                         pa_tensor block_mapping, const pa_opts *opts) {
  pa_opts o;
  std::memset(&o, 0, sizeof o);
  if (opts) o = *opts;
  pa_status st;
  const pa_tensor *pools[4] = {&dst_k_cache, &dst_v_cache, &src_k_cache, &src_v_cache};
  const char *names[4] = {"dst_k_cache", "dst_v_cache", "src_k_cache", "src_v_cache"};
  for (int i = 0; i < 4; ++i)
    if ((st = check_tensor(*pools[i], names[i], 4, true))) return st;
  if ((st = check_tensor(block_mapping, "block_mapping", 2, false))) return st;
  if (block_mapping.dtype != PA_I64 && block_mapping.dtype != PA_I32)
    return fail(PA_ERR_DTYPE, "block_mapping: dtype must be I64 or I32");
  if (block_mapping.shape[1] != 2) return fail(PA_ERR_SHAPE, "block_mapping must be [num_pairs, 2]");
  const int eb = elem_bytes(src_k_cache.dtype);
  for (int i = 0; i < 4; ++i) {
    const pa_tensor &t = *pools[i];
    if (t.dtype != src_k_cache.dtype) return fail(PA_ERR_DTYPE, "%s: dtype differs from src_k_cache", names[i]);
    for (int j = 1; j < 4; ++j)
      if (t.shape[j] != src_k_cache.shape[j])
        return fail(PA_ERR_SHAPE, "%s: block shape differs from src_k_cache in dim %d", names[i], j);
    if (t.stride[2] != t.shape[3] || t.stride[1] != t.shape[2] * t.shape[3])
      return fail(PA_ERR_LAYOUT, "%s: each block must be one contiguous run", names[i]);
  }
  if (dst_k_cache.shape[0] != dst_v_cache.shape[0] || src_k_cache.shape[0] != src_v_cache.shape[0])
    return fail(PA_ERR_SHAPE, "K and V pools of one side must have the same number of blocks");
  if (dst_k_cache.stride[0] != dst_v_cache.stride[0] || src_k_cache.stride[0] != src_v_cache.stride[0])
    return fail(PA_ERR_LAYOUT, "K and V pools of one side must have the same block stride");
  if ((st = check_flags(o))) return st;
  const int64_t M = block_mapping.shape[0];
  const int64_t block_bytes = src_k_cache.shape[1] * src_k_cache.shape[2] * src_k_cache.shape[3] * eb;
  if (M == 0 || block_bytes == 0 || src_k_cache.shape[0] == 0 || dst_k_cache.shape[0] == 0) return PA_OK;
  if (block_bytes % 16) return fail(PA_ERR_LAYOUT, "a block of %lld bytes is not a whole number of 16-byte vectors",
                                    (long long)block_bytes);
  const int64_t pieces = pa::copy_blocks_pieces(block_bytes);
  if (M * 2 * pieces > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "too many block pairs");
  if (block_mapping.stride[1] != 1) return fail(PA_ERR_LAYOUT, "block_mapping: pairs must be contiguous");

  pa::BlockCopyArgs a;
  std::memset(&a, 0, sizeof a);
  void *dev[5];
  const void *ptrs[5] = {dst_k_cache.data, dst_v_cache.data, src_k_cache.data, src_v_cache.data, block_mapping.data};
  const char *pnames[5] = {"dst_k_cache", "dst_v_cache", "src_k_cache", "src_v_cache", "block_mapping"};
  for (int i = 0; i < 5; ++i)
    if ((st = device_address(ptrs[i], pnames[i], &dev[i]))) return st;
  if (o.flags & PA_FLAG_VALIDATE) {
    const hipStream_t stream = static_cast<hipStream_t>(o.stream);
    pa::HostInts pairs;
    if ((st = pa::validation_allowed(stream))) return st;
    if ((st = pairs.fetch(block_mapping, "block_mapping", stream))) return st;
    const bool same_pool = dst_k_cache.data == src_k_cache.data || dst_v_cache.data == src_v_cache.data;
    if ((st = pa::check_block_pairs(pairs, src_k_cache.shape[0], dst_k_cache.shape[0], same_pool))) return st;
  }
  a.dst_k = static_cast<char *>(dev[0]);
  a.dst_v = static_cast<char *>(dev[1]);
  a.src_k = static_cast<const char *>(dev[2]);
  a.src_v = static_cast<const char *>(dev[3]);
  a.mapping = dev[4];
  a.map_i64 = block_mapping.dtype == PA_I64;
  a.map_stride = block_mapping.stride[0];
  a.num_pairs = M;
  a.block_bytes = block_bytes;
  a.src_stride = src_k_cache.stride[0] * eb;
  a.dst_stride = dst_k_cache.stride[0] * eb;
  a.src_blocks = src_k_cache.shape[0];
  a.dst_blocks = dst_k_cache.shape[0];
  a.pieces = (int32_t)pieces;
  hipError_t e = pa::launch_copy_blocks(a, static_cast<hipStream_t>(o.stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "block-copy kernel launch: %s", hipGetErrorString(e));
  return PA_OK;
}

pa_status pa_stream_read(const void *buf, int64_t bytes, int32_t num_workgroups, int32_t loads_in_flight,
                         int32_t nontemporal, uint32_t *partials, const pa_opts *opts) {
  pa_opts o;
  std::memset(&o, 0, sizeof o);
  if (opts) o = *opts;
  pa_status st;
  if (!buf || !partials) return fail(PA_ERR_NULL, "buf and partials are required");
  if ((st = check_flags(o))) return st;
  if (o.flags & PA_FLAG_VALIDATE) return fail(PA_ERR_ARG, "pa_stream_read: PA_FLAG_VALIDATE has nothing to check");
  if (bytes <= 0 || bytes % 16) return fail(PA_ERR_SHAPE, "bytes must be a positive multiple of 16, got %lld",
                                            (long long)bytes);
  if (reinterpret_cast<uintptr_t>(buf) % 16) return fail(PA_ERR_LAYOUT, "buf must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(partials) % 4) return fail(PA_ERR_LAYOUT, "partials must be 4-byte aligned");
  if (num_workgroups < 1 || num_workgroups > 65536)
    return fail(PA_ERR_ARG, "num_workgroups must be in [1, 65536], got %d", num_workgroups);
  if (loads_in_flight != 1 && loads_in_flight != 4 && loads_in_flight != 8)
    return fail(PA_ERR_UNSUPPORTED, "loads_in_flight must be 1, 4 or 8, got %d", loads_in_flight);
  void *db, *dp;
  if ((st = device_address(buf, "buf", &db))) return st;
  if ((st = device_address(partials, "partials", &dp))) return st;
  hipError_t e = pa::launch_stream_read(db, bytes, num_workgroups, loads_in_flight, nontemporal != 0,
                                        static_cast<uint32_t *>(dp), static_cast<hipStream_t>(o.stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "stream-read kernel launch: %s", hipGetErrorString(e));
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
    case PA_ERR_BAD_INDEX: return "index or scale entry out of range";
  }
  return "unknown status";
}

const char *pa_last_error(void) { return g_last_error; }

const char *pa_version(void) { return "0.3.0"; }

}  // extern "C"
