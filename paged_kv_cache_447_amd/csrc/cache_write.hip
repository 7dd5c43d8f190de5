// Scatter of new tokens' K/V rows into the paged cache.
//
// Token n goes to physical slot slot_mapping[n]: block slot / block_size,
// offset slot % block_size (the address rule physical = block * page size +
// offset of page "Paged KVCache：大模型推理显存管理优化方案", section 2.3, with the
// page counted in tokens).  A decode step appends one token per sequence; the
// scheduler sketched in section 3.1 of page
// "vLLM推理引擎架构：PagedAttention机制与高吞吐推理" allocates a fresh block when a
// sequence crosses a block boundary, so the slot may be the first of a block.
//
// In the [num_blocks, block_size, num_kv_heads, head_dim] layout the
// destination of one token, all heads, is a contiguous num_kv_heads * head_dim
// run, so the copy is a straight 16-byte-vector copy.  One workgroup per
// (token, K or V).  fp8 caches quantise on the way: x / scale in fp32, then
// round to the nearest e4m3fn value, ties to even, saturating at +-448.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kThreads = 256;

// fp32 -> OCP e4m3fn (bias 7, 3 mantissa bits, max 448, NaN = S.1111.111),
// round to nearest even, saturating.
__device__ __forceinline__ uint32_t f32_to_e4m3fn_sat(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (u >> 24) & 0x80u;
  u &= 0x7FFFFFFFu;
  if (u > 0x7F800000u) return sign | 0x7Fu;   // NaN
  if (u >= 0x43E00000u) return sign | 0x7Eu;  // |x| >= 448, infinities included
  if (u < 0x3C800000u) {                      // |x| < 2^-6: subnormal grid of step 2^-9
    const float steps = __builtin_bit_cast(float, u) * 512.0f;  // exact scaling
    return sign | (uint32_t)__builtin_rintf(steps);             // 8 lands on the smallest normal
  }
  // normal range: keep 3 mantissa bits, round the 20 dropped bits to nearest even
  const uint32_t e = (u >> 23) - 120u;  // rebias 127 -> 7
  const uint32_t mant = u & 0x7FFFFFu;
  uint32_t code = (e << 3) | (mant >> 20);
  const uint32_t rest = mant & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (code & 1u))) code += 1u;  // carry may bump the exponent
  return sign | code;
}

template <typename T>
__device__ __forceinline__ int64_t read_slot(const void *p, int n);
template <>
__device__ __forceinline__ int64_t read_slot<int64_t>(const void *p, int n) {
  return reinterpret_cast<const int64_t *>(p)[n];
}
template <>
__device__ __forceinline__ int64_t read_slot<int32_t>(const void *p, int n) {
  return reinterpret_cast<const int32_t *>(p)[n];
}

// same dtype in and out: a byte copy in 16-byte vectors
template <typename SlotT, int EBYTES>
__global__ void __launch_bounds__(kThreads) cache_copy_kernel(const CacheWriteArgs a) {
  const int n = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  const int64_t slot = read_slot<SlotT>(a.slot_mapping, n);
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot / a.block_size, off = slot % a.block_size;
  const char *src = reinterpret_cast<const char *>(is_v ? a.v : a.k);
  char *dst = reinterpret_cast<char *>(is_v ? a.v_cache : a.k_cache);
  const int64_t s_n = is_v ? a.v_sn : a.k_sn, s_h = is_v ? a.v_sh : a.k_sh;
  const int64_t c_b = is_v ? a.vc_sb : a.kc_sb, c_t = is_v ? a.vc_st : a.kc_st, c_h = is_v ? a.vc_sh : a.kc_sh;
  constexpr int VEC = 16 / EBYTES;
  const int per_head = a.head_dim / VEC;
  const int total = a.num_kv_heads * per_head;
  for (int i = threadIdx.x; i < total; i += kThreads) {
    const int h = i / per_head, c = (i % per_head) * VEC;
    const u32x4 w = ld16(src + ((int64_t)n * s_n + (int64_t)h * s_h + c) * EBYTES);
    st16(dst + (blk * c_b + off * c_t + (int64_t)h * c_h + c) * EBYTES, w);
  }
}

// fp8 cache: 16 output codes (one 16-byte store) per thread and step
template <typename SlotT, typename InT>
__global__ void __launch_bounds__(kThreads) cache_quant_kernel(const CacheWriteArgs a) {
  const int n = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  const int64_t slot = read_slot<SlotT>(a.slot_mapping, n);
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot / a.block_size, off = slot % a.block_size;
  const void *src = is_v ? a.v : a.k;
  char *dst = reinterpret_cast<char *>(is_v ? a.v_cache : a.k_cache);
  const int64_t s_n = is_v ? a.v_sn : a.k_sn, s_h = is_v ? a.v_sh : a.k_sh;
  const int64_t c_b = is_v ? a.vc_sb : a.kc_sb, c_t = is_v ? a.vc_st : a.kc_st, c_h = is_v ? a.vc_sh : a.kc_sh;
  const float *head_scale = is_v ? a.v_head_scale : a.k_head_scale;  // null: one scale for the tensor
  // per (block, kv head): the scales of this token's destination block, else null
  const float *block_scale = is_v ? a.v_block_scale : a.k_block_scale;
  if (block_scale) block_scale += blk * a.num_kv_heads;
  const float tensor_scale = is_v ? a.v_scale : a.k_scale;
  const int per_head = a.head_dim / 16;
  const int total = a.num_kv_heads * per_head;
  for (int i = threadIdx.x; i < total; i += kThreads) {
    const int h = i / per_head, c = (i % per_head) * 16;
    const float scale = block_scale ? block_scale[h] : (head_scale ? head_scale[h] : tensor_scale);
    const int64_t sb = (int64_t)n * s_n + (int64_t)h * s_h + c;
    constexpr int IVEC = Elem<InT>::kPer16;
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; j += IVEC) {
      const u32x4 w = ld16(reinterpret_cast<const char *>(src) + (sb + j) * Elem<InT>::kBytes);
      Elem<InT>::unpack(w, x + j);
    }
    u32x4 out;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) word |= f32_to_e4m3fn_sat(x[4 * k + b] / scale) << (8 * b);
      out[k] = word;
    }
    st16(dst + blk * c_b + off * c_t + (int64_t)h * c_h + c, out);
  }
}

template <typename SlotT>
hipError_t launch_typed(const CacheWriteArgs &a, hipStream_t stream) {
  dim3 grid(a.num_tokens, 2);
  dim3 block(kThreads);
  if (a.cache_kind == KV_FP8) {
    switch (a.in_kind) {
      case KV_F32: hipLaunchKernelGGL((cache_quant_kernel<SlotT, f32_t>), grid, block, 0, stream, a); break;
      case KV_F16: hipLaunchKernelGGL((cache_quant_kernel<SlotT, f16_t>), grid, block, 0, stream, a); break;
      case KV_BF16: hipLaunchKernelGGL((cache_quant_kernel<SlotT, bf16_t>), grid, block, 0, stream, a); break;
      case KV_FP8: hipLaunchKernelGGL((cache_copy_kernel<SlotT, 1>), grid, block, 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.cache_kind) {
      case KV_F32: hipLaunchKernelGGL((cache_copy_kernel<SlotT, 4>), grid, block, 0, stream, a); break;
      case KV_F16:
      case KV_BF16: hipLaunchKernelGGL((cache_copy_kernel<SlotT, 2>), grid, block, 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs &a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  return a.slot_i64 ? launch_typed<int64_t>(a, stream) : launch_typed<int32_t>(a, stream);
}

}  // namespace pa
