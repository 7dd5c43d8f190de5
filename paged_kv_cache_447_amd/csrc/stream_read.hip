// A plain streaming read of one buffer, for measurement: the practical HBM
// read rate on this part, against which the decode kernels' K/V streams are
// compared (they read every byte of their K/V rows once, as this does).  No
// step of the attention path runs here.
//
// Each thread walks the buffer grid-stride in 16-byte vectors with LOADS of
// them in flight before any is used, folds them into an XOR checksum, and each
// workgroup writes one 32-bit partial (the XOR of every word it read), so the
// loads cannot be dropped and the result can be checked exactly.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kThreads = 256;

template <int LOADS, bool NT>
__global__ void __launch_bounds__(kThreads)
    stream_read_kernel(const u32x4 *__restrict__ p, uint64_t n16, uint32_t *__restrict__ partials) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  // every vector of a batch is in bounds: the last is at i + (LOADS - 1) * stride < n16
  for (; i + (LOADS - 1) * stride < n16; i += LOADS * stride) {
    u32x4 v[LOADS];
#pragma unroll
    for (int u = 0; u < LOADS; ++u) v[u] = NT ? ld16_stream(p + i + u * stride) : ld16(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < LOADS; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = ld16(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t s[kThreads];
  s[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < kThreads; ++t) r ^= s[t];
    partials[blockIdx.x] = r;
  }
}

template <int LOADS>
void launch_loads(const u32x4 *p, uint64_t n16, int wgs, bool nt, uint32_t *partials, hipStream_t stream) {
  if (nt)
    hipLaunchKernelGGL((stream_read_kernel<LOADS, true>), dim3(wgs), dim3(kThreads), 0, stream, p, n16, partials);
  else
    hipLaunchKernelGGL((stream_read_kernel<LOADS, false>), dim3(wgs), dim3(kThreads), 0, stream, p, n16, partials);
}

}  // namespace

hipError_t launch_stream_read(const void *buf, int64_t bytes, int workgroups, int loads, bool nontemporal,
                              uint32_t *partials, hipStream_t stream) {
  const u32x4 *p = static_cast<const u32x4 *>(buf);
  const uint64_t n16 = (uint64_t)bytes / 16;
  switch (loads) {
    case 1: launch_loads<1>(p, n16, workgroups, nontemporal, partials, stream); break;
    case 4: launch_loads<4>(p, n16, workgroups, nontemporal, partials, stream); break;
    case 8: launch_loads<8>(p, n16, workgroups, nontemporal, partials, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
