// PA_FLAG_VALIDATE: the checks a call runs, when asked, on the index and
// scale arrays it would otherwise trust.  The kernels never follow an entry
// out of bounds (they clamp), but a table entry outside the pool, a context
// longer than its table, or two tokens written to one slot make a result
// unspecified.  The pages treat such entries as faults to be reported to the
// owner of the mapping: an unmapped page-table entry raises a page fault
// (page "Paged KVCache：大模型推理显存管理优化方案", section 2.3, address
// translation), and an allocation the pool cannot serve raises an error
// (page "vLLM推理引擎架构：PagedAttention机制与高吞吐推理", section 2.2, the
// block manager).  Here the call copies the arrays to the host after the
// stream's earlier work, checks them, and returns PA_ERR_BAD_INDEX naming the
// first bad entry before anything is enqueued.
#include "pa_validate.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <unordered_map>
#include <unordered_set>

namespace pa {
pa_status fail_message(pa_status s, const char *msg);
}

namespace {

pa_status failf(pa_status s, const char *fmt, ...) {
  char msg[400];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, sizeof msg, fmt, ap);
  va_end(ap);
  return pa::fail_message(s, msg);
}

// Bytes from device or pinned host memory into `dst`, ordered after the
// stream's earlier work; waits for the copy.
pa_status copy_to_host(void *dst, const void *src, size_t bytes, hipStream_t stream, const char *name) {
  if (bytes == 0) return PA_OK;
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDefault, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return failf(PA_ERR_HIP, "PA_FLAG_VALIDATE: copying %s to the host: %s", name, hipGetErrorString(e));
  }
  return PA_OK;
}

}  // namespace

namespace pa {

pa_status validation_allowed(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return failf(PA_ERR_HIP, "PA_FLAG_VALIDATE: querying the stream's capture state: %s", hipGetErrorString(e));
  }
  if (cs != hipStreamCaptureStatusNone)
    return failf(PA_ERR_ARG, "PA_FLAG_VALIDATE copies to the host and waits: not allowed on a capturing stream");
  return PA_OK;
}

pa_status HostInts::fetch(const pa_tensor &t, const char *name, hipStream_t stream) {
  rows = t.shape[0];
  cols = t.ndim == 2 ? t.shape[1] : 1;
  v.assign((size_t)(rows * cols), 0);
  if (rows == 0 || cols == 0) return PA_OK;
  const int eb = t.dtype == PA_I64 ? 8 : 4;
  const int64_t s0 = t.stride[0], s1 = t.ndim == 2 ? t.stride[1] : 0;
  const int64_t span = (rows - 1) * s0 + (cols - 1) * s1 + 1;  // elements from the first to the last
  std::vector<char> raw((size_t)(span * eb));
  pa_status st = copy_to_host(raw.data(), t.data, raw.size(), stream, name);
  if (st) return st;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      const char *p = raw.data() + (r * s0 + c * s1) * eb;
      int64_t x;
      if (eb == 8) {
        std::memcpy(&x, p, 8);
      } else {
        int32_t y;
        std::memcpy(&y, p, 4);
        x = y;
      }
      v[(size_t)(r * cols + c)] = x;
    }
  return PA_OK;
}

pa_status check_tables(const HostInts &bt, const HostInts &lens, int64_t block_size, int64_t num_blocks) {
  const int64_t max_ctx = bt.cols * block_size;
  for (int64_t s = 0; s < lens.rows; ++s) {
    const int64_t L = lens.at(s);
    if (L < 0 || L > max_ctx)
      return failf(PA_ERR_BAD_INDEX, "context_lens[%lld] = %lld outside [0, %lld] (max_blocks_per_seq * block_size)",
                   (long long)s, (long long)L, (long long)max_ctx);
    for (int64_t j = 0; j < (L + block_size - 1) / block_size; ++j) {
      const int64_t b = bt.at(s, j);
      if (b < 0 || b >= num_blocks)
        return failf(PA_ERR_BAD_INDEX, "block_tables[%lld][%lld] = %lld outside [0, %lld) (a block of the context)",
                     (long long)s, (long long)j, (long long)b, (long long)num_blocks);
    }
  }
  return PA_OK;
}

pa_status check_new_token_slots(const HostInts &slots, const HostInts &bt, const HostInts &lens, int64_t block_size,
                                int64_t num_slots) {
  std::unordered_set<int64_t> seen;
  for (int64_t s = 0; s < slots.rows; ++s) {
    const int64_t slot = slots.at(s), L = lens.at(s);
    if (slot < 0 || slot >= num_slots || L <= 0) continue;  // skipped: nothing written
    const int64_t want = bt.at(s, (L - 1) / block_size) * block_size + (L - 1) % block_size;
    if (slot != want)
      return failf(PA_ERR_BAD_INDEX, "slot_mapping[%lld] = %lld is not the slot of position %lld (%lld)",
                   (long long)s, (long long)slot, (long long)(L - 1), (long long)want);
    if (!seen.insert(slot).second)
      return failf(PA_ERR_BAD_INDEX, "slot_mapping[%lld] = %lld is also another sequence's slot", (long long)s,
                   (long long)slot);
  }
  return PA_OK;
}

pa_status check_distinct_slots(const HostInts &slots, int64_t num_slots) {
  std::unordered_map<int64_t, int64_t> first;
  for (int64_t n = 0; n < slots.rows; ++n) {
    const int64_t slot = slots.at(n);
    if (slot < 0 || slot >= num_slots) continue;  // skipped
    auto it = first.emplace(slot, n);
    if (!it.second)
      return failf(PA_ERR_BAD_INDEX, "slot_mapping[%lld] = slot_mapping[%lld] = %lld: slots must be distinct",
                   (long long)it.first->second, (long long)n, (long long)slot);
  }
  return PA_OK;
}

pa_status check_query_starts(const HostInts &qsl, const HostInts &lens, int64_t num_rows) {
  if (qsl.rows == 0) return PA_OK;
  if (qsl.at(0) != 0) return failf(PA_ERR_BAD_INDEX, "query_start_loc[0] = %lld, must be 0", (long long)qsl.at(0));
  for (int64_t s = 0; s + 1 < qsl.rows; ++s) {
    const int64_t n = qsl.at(s + 1) - qsl.at(s);
    if (n < 0 || qsl.at(s + 1) > num_rows)
      return failf(PA_ERR_BAD_INDEX, "query_start_loc[%lld] = %lld: not non-decreasing within [0, %lld]",
                   (long long)(s + 1), (long long)qsl.at(s + 1), (long long)num_rows);
    if (n > lens.at(s))
      return failf(PA_ERR_BAD_INDEX, "sequence %lld has %lld query rows but a context of %lld tokens", (long long)s,
                   (long long)n, (long long)lens.at(s));
  }
  if (qsl.at(qsl.rows - 1) != num_rows)
    return failf(PA_ERR_BAD_INDEX, "query_start_loc[%lld] = %lld, must be num_tokens = %lld", (long long)(qsl.rows - 1),
                 (long long)qsl.at(qsl.rows - 1), (long long)num_rows);
  return PA_OK;
}

pa_status check_block_pairs(const HostInts &map, int64_t src_blocks, int64_t dst_blocks, bool same_pool) {
  std::unordered_map<int64_t, int64_t> dst_pair;
  std::unordered_set<int64_t> sources;
  for (int64_t i = 0; i < map.rows; ++i) {
    const int64_t s = map.at(i, 0), d = map.at(i, 1);
    if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks) continue;  // skipped
    auto it = dst_pair.emplace(d, i);
    if (!it.second)
      return failf(PA_ERR_BAD_INDEX, "pairs %lld and %lld both write destination block %lld",
                   (long long)it.first->second, (long long)i, (long long)d);
    sources.insert(s);
  }
  if (same_pool)
    for (const auto &kv : dst_pair)
      if (sources.count(kv.first))
        return failf(PA_ERR_BAD_INDEX, "block %lld is a destination (pair %lld) and a source in one pool",
                     (long long)kv.first, (long long)kv.second);
  return PA_OK;
}

pa_status check_head_scales(const float *k_head_scales, const float *v_head_scales, int64_t n, hipStream_t stream,
                            const char *k_name, const char *v_name) {
  if (!k_head_scales || n <= 0) return PA_OK;
  std::vector<float> h((size_t)n);
  const float *src[2] = {k_head_scales, v_head_scales};
  const char *names[2] = {k_name, v_name};
  for (int i = 0; i < 2; ++i) {
    pa_status st = copy_to_host(h.data(), src[i], (size_t)n * sizeof(float), stream, names[i]);
    if (st) return st;
    for (int64_t j = 0; j < n; ++j)
      if (!(h[(size_t)j] > 0.0f) || !std::isfinite(h[(size_t)j]))
        return failf(PA_ERR_BAD_INDEX, "%s[%lld] = %g: scales must be finite and > 0", names[i], (long long)j,
                     (double)h[(size_t)j]);
  }
  return PA_OK;
}

}  // namespace pa
