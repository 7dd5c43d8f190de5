// Whole-block copies between two paged pools, driven by a list of
// (source block, destination block) pairs.
//
// Two uses on the pages: copy-on-write, where a sequence about to write into
// a block it shares with others first gets a private copy of it (page
// "vLLM框架中的KV cache优化与PagedAttention机制详解", section 5.1, step 4: shared
// blocks are copied before they are modified), and swapping, where whole
// blocks move between GPU memory and host memory when sequences are preempted
// and resumed (page "Paged KVCache：大模型推理显存管理优化方案", section 5, pages
// migrating between memory tiers; page "vLLM推理引擎架构：PagedAttention机制与高吞吐推理",
// section 3.1, the CPU swap space).  Both pools may live in device memory or
// in pinned, device-mapped host memory: the same kernel then reads or writes
// across the host link.
//
// A block of [block_size, num_kv_heads, head_dim] elements is one contiguous
// run of bytes in this cache layout, so a copy is a straight 16-byte-vector
// stream: one workgroup per (pair, K or V, 16 KB piece of the block), every
// lane moving 16 bytes per step, loads and stores marked non-temporal (each
// byte is touched once).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kPieceBytes = (int64_t)kThreads * 16 * kUnroll;  // 16 KB

__global__ void __launch_bounds__(kThreads) copy_blocks_kernel(const BlockCopyArgs a) {
  const int64_t id = blockIdx.x;
  const int64_t per_pair = 2 * (int64_t)a.pieces;
  const int64_t pair = id / per_pair;
  const int rem = (int)(id - pair * per_pair);
  const int isv = rem / a.pieces, piece = rem - isv * a.pieces;
  int64_t s, d;
  if (a.map_i64) {
    const int64_t *m = reinterpret_cast<const int64_t *>(a.mapping) + pair * a.map_stride;
    s = m[0];
    d = m[1];
  } else {
    const int32_t *m = reinterpret_cast<const int32_t *>(a.mapping) + pair * a.map_stride;
    s = m[0];
    d = m[1];
  }
  // pairs naming no block of their pool are skipped, never followed
  if (s < 0 || d < 0 || s >= a.src_blocks || d >= a.dst_blocks) return;
  const char *src = (isv ? a.src_v : a.src_k) + s * a.src_stride;
  char *dst = (isv ? a.dst_v : a.dst_k) + d * a.dst_stride;
  const int64_t lo = piece * kPieceBytes;
  const int64_t n = min(kPieceBytes, a.block_bytes - lo);  // bytes of this piece, a multiple of 16
  u32x4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t off = lo + 16 * ((int64_t)u * kThreads + threadIdx.x);
    if (off - lo < n) v[u] = ld16_stream(src + off);
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t off = lo + 16 * ((int64_t)u * kThreads + threadIdx.x);
    if (off - lo < n) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4 *>(dst + off));
  }
}

}  // namespace

int64_t copy_blocks_pieces(int64_t block_bytes) { return (block_bytes + kPieceBytes - 1) / kPieceBytes; }

hipError_t launch_copy_blocks(const BlockCopyArgs &a, hipStream_t stream) {
  const int64_t wgs = a.num_pairs * 2 * (int64_t)a.pieces;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
