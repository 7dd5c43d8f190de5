// pa_decode_static: pa_decode for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
// The decode workspace -- merge counters and partial-result slots -- lives
// in a file-scope device array of a fixed size instead of caller memory.
//
// The array's name is a host-side stand-in, not a device address: its
// address on each device is looked up once, with that device current, by
// hipGetSymbolAddress, and only that address reaches the kernels.  At that
// first use on a device the array is cleared by a fill kernel on the
// caller's stream; every decode leaves its counters (at the array's end) at
// zero again and garbage only in its partial-result slots (from the array's
// start, an extent fixed by the head shape and worker count), so later calls
// of any batch size find their counters cleared.  A call whose counters would
// reach into slots an earlier call used (another head shape or worker count)
// clears the array again first.  Every call on one device shares that
// device's array: calls that overlap on one device race.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "pa.h"
#include "pa_internal.h"

namespace pa {
size_t decode_partials_bytes(int64_t num_heads, int64_t num_kv_heads, int64_t head_dim, int32_t num_workers);
pa_status decode_with_workspace(pa_tensor out, pa_tensor q, pa_tensor k_cache, pa_tensor v_cache,
                                pa_tensor block_tables, pa_tensor context_lens, int32_t block_size, float scale,
                                int32_t num_kv_heads, const pa_opts *opts, void *workspace, size_t workspace_bytes);
pa_status fail_message(pa_status s, const char *msg);
}  // namespace pa

namespace {

constexpr size_t kScratchBytes = size_t(24) << 20;  // 24 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void clear_scratch(uint4 *p, size_t n) {
  const uint4 z = {0u, 0u, 0u, 0u};
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = z;
}

std::mutex g_mu;
void *g_ptr[kMaxDevices];     // device address of `scratch` on each device, once looked up
size_t g_dirty[kMaxDevices];  // bytes from the array's start that calls since its last clear may have left non-zero

pa_status enqueue_clear(void *ptr, hipStream_t stream) {
  hipLaunchKernelGGL(clear_scratch, dim3(256), dim3(256), 0, stream, static_cast<uint4 *>(ptr),
                     kScratchBytes / sizeof(uint4));
  const hipError_t le = hipGetLastError();
  if (le != hipSuccess) {
    char msg[160];
    snprintf(msg, sizeof msg, "clearing the static scratch: %s", hipGetErrorString(le));
    return pa::fail_message(PA_ERR_HIP, msg);
  }
  return PA_OK;
}

// The scratch of the current device for a call whose counters start
// `counters_from` bytes into it and whose slots end `parts` bytes into it:
// its address (looked up and cleared on the device's first call; cleared
// again if the counters would overlap slots earlier calls used; clears
// enqueued on `stream`), or null with the error message set.
void *device_scratch(hipStream_t stream, size_t counters_from, size_t parts, pa_status *st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    *st = pa::fail_message(PA_ERR_HIP, "no current HIP device for the static scratch");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev]) {
    if (counters_from < g_dirty[dev]) {
      if ((*st = enqueue_clear(g_ptr[dev], stream)) != PA_OK) return nullptr;
      g_dirty[dev] = 0;
    }
    if (parts > g_dirty[dev]) g_dirty[dev] = parts;
    return g_ptr[dev];
  }
  void *ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    (void)hipGetLastError();
    char msg[160];
    snprintf(msg, sizeof msg, "hipGetSymbolAddress of the static scratch: %s", hipGetErrorString(e));
    *st = pa::fail_message(PA_ERR_HIP, msg);
    return nullptr;
  }
  if ((*st = enqueue_clear(ptr, stream)) != PA_OK) return nullptr;
  g_ptr[dev] = ptr;
  g_dirty[dev] = parts;
  return ptr;
}

}  // namespace

extern "C" {

size_t pa_decode_static_scratch_bytes(void) { return kScratchBytes; }

pa_status pa_decode_static(pa_tensor out, pa_tensor q, pa_tensor k_cache, pa_tensor v_cache, pa_tensor block_tables,
                           pa_tensor context_lens, int32_t block_size, float scale, int32_t num_kv_heads,
                           const pa_opts *opts) {
  if (opts && (opts->workspace || opts->workspace_bytes))
    return pa::fail_message(PA_ERR_ARG, "opts->workspace must be NULL: this entry point uses the library's own scratch");
  // refuse requests past the scratch before anything touches a device
  const int64_t S = q.ndim == 3 ? q.shape[0] : 0, H = q.ndim == 3 ? q.shape[1] : 0, D = q.ndim == 3 ? q.shape[2] : 0;
  const int32_t workers = opts ? opts->num_workers : 0;
  size_t need = 0, parts = 0;
  if (S > 0 && H > 0 && num_kv_heads > 0 && H % num_kv_heads == 0) {
    need = pa_decode_workspace_size(S, H, num_kv_heads, D, workers);
    parts = pa::decode_partials_bytes(H, num_kv_heads, D, workers);
    if (need > kScratchBytes) {
      char msg[200];
      snprintf(msg, sizeof msg, "this decode needs %zu bytes of workspace; the static scratch holds %zu", need,
               kScratchBytes);
      return pa::fail_message(PA_ERR_WORKSPACE, msg);
    }
  }
  pa_status st = PA_OK;
  // the counters take the array's last (need - parts) bytes
  void *ws = device_scratch(static_cast<hipStream_t>(opts ? opts->stream : nullptr), kScratchBytes - (need - parts),
                            parts, &st);
  if (!ws) return st;
  return pa::decode_with_workspace(out, q, k_cache, v_cache, block_tables, context_lens, block_size, scale,
                                   num_kv_heads, opts, ws, kScratchBytes);
}

}  // extern "C"
