// Device-side helpers shared by the gfx950 kernels: 16-byte vector loads,
// element unpacking, wave64 lane reductions through DPP.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
// K/V rows are read once per launch: nontemporal loads mark them as streaming
// data, which on gfx950 keeps them from displacing reusable lines and lets
// the memory system stream at a markedly higher rate than plain loads.
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

// ---------------------------------------------------------------------------------
// storage element types

struct f32_t { using storage = float; };
struct f16_t { using storage = _Float16; };
struct bf16_t { using storage = uint16_t; };
struct fp8_t { using storage = uint8_t; };

template <typename T> struct Elem;

template <> struct Elem<f32_t> {
  static constexpr int kBytes = 4;
  static constexpr int kPer16 = 4;
  __device__ static void unpack(u32x4 w, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // copy the lane out first: a bit cast applied directly to a vector
      // element is lowered as a read of element 0
      const uint32_t x = w[i];
      f[i] = __builtin_bit_cast(float, x);
    }
  }
  __device__ static float load(const void *p, int64_t i) { return reinterpret_cast<const float *>(p)[i]; }
  __device__ static void store(void *p, int64_t i, float x) { reinterpret_cast<float *>(p)[i] = x; }
};

template <> struct Elem<f16_t> {
  static constexpr int kBytes = 2;
  static constexpr int kPer16 = 8;
  __device__ static void unpack(u32x4 w, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
      f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    }
  }
  __device__ static float load(const void *p, int64_t i) { return (float)reinterpret_cast<const _Float16 *>(p)[i]; }
  __device__ static void store(void *p, int64_t i, float x) { reinterpret_cast<_Float16 *>(p)[i] = (_Float16)x; }
};

// bf16 <-> f32: the bf16 bits are the upper half of the f32 bits; f32 -> bf16
// rounds to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <> struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  static constexpr int kPer16 = 8;
  __device__ static void unpack(u32x4 w, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
  }
  __device__ static float load(const void *p, int64_t i) {
    return __builtin_bit_cast(float, (uint32_t)reinterpret_cast<const uint16_t *>(p)[i] << 16);
  }
  __device__ static void store(void *p, int64_t i, float x) { reinterpret_cast<uint16_t *>(p)[i] = f32_to_bf16_rne(x); }
};

// OCP e4m3fn codes; gfx950's v_cvt_pk_f32_fp8 decodes the OCP format.
template <> struct Elem<fp8_t> {
  static constexpr int kBytes = 1;
  static constexpr int kPer16 = 16;
  __device__ static void unpack(u32x4 w, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
      auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
      f[4 * i] = lo[0];
      f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0];
      f[4 * i + 3] = hi[1];
    }
  }
};

// Two e4m3fn codes of a 32-bit word (bytes 0-1, or 2-3 with `hi`) to a packed
// pair of f16 or bf16 values.  Exact: every e4m3fn value is representable in
// both 16-bit formats (gfx950 converts with a unit scale).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// ---------------------------------------------------------------------------------
// wave64 lane exchange

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

enum : int {
  DPP_QUAD_XOR1 = 0xB1,   // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,   // quad_perm [2,3,0,1]
  DPP_ROW_ROR4 = 0x124,   // rotate right by 4 within a 16-lane row
  DPP_ROW_ROR8 = 0x128,   // rotate right by 8 within a 16-lane row
  DPP_ROW_MIRROR = 0x140, // lane i <- lane 15-i within a row
  DPP_ROW_HALF_MIRROR = 0x141,  // lane i <- lane 7-i within each half row
};

// Sum over aligned groups of N consecutive lanes (N = 1..32); every lane of a group
// receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<DPP_QUAD_XOR1>(v);
  if constexpr (N >= 4) v += dpp<DPP_QUAD_XOR2>(v);
  if constexpr (N >= 8) v += dpp<DPP_ROW_HALF_MIRROR>(v);
  if constexpr (N >= 16) v += dpp<DPP_ROW_MIRROR>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  return v;
}

// The same for M independent values, one DPP step across all of them at a
// time, so that no step waits on the one before it for the same value.
template <int N, int M>
__device__ __forceinline__ void group_sum_n(float *v) {
  if constexpr (N >= 2) {
#pragma unroll
    for (int i = 0; i < M; ++i) v[i] += dpp<DPP_QUAD_XOR1>(v[i]);
  }
  if constexpr (N >= 4) {
#pragma unroll
    for (int i = 0; i < M; ++i) v[i] += dpp<DPP_QUAD_XOR2>(v[i]);
  }
  if constexpr (N >= 8) {
#pragma unroll
    for (int i = 0; i < M; ++i) v[i] += dpp<DPP_ROW_HALF_MIRROR>(v[i]);
  }
  if constexpr (N >= 16) {
#pragma unroll
    for (int i = 0; i < M; ++i) v[i] += dpp<DPP_ROW_MIRROR>(v[i]);
  }
  if constexpr (N >= 32) {
#pragma unroll
    for (int i = 0; i < M; ++i) v[i] += __shfl_xor(v[i], 16);
  }
}

// Combine across the 64/N groups of N lanes (lanes at the same position in every
// group end up with the same result).  N is a power of two, 4 <= N <= 32.
template <int N>
__device__ __forceinline__ float across_groups_max(float v) {
  if constexpr (N <= 4) v = fmaxf(v, dpp<DPP_ROW_ROR4>(v));
  if constexpr (N <= 8) v = fmaxf(v, dpp<DPP_ROW_ROR8>(v));
  if constexpr (N <= 16) v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

template <int N>
__device__ __forceinline__ float across_groups_sum(float v) {
  if constexpr (N <= 4) v += dpp<DPP_ROW_ROR4>(v);
  if constexpr (N <= 8) v += dpp<DPP_ROW_ROR8>(v);
  if constexpr (N <= 16) v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp<DPP_QUAD_XOR2>(v));
  v = fmaxf(v, dpp<DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_ROW_MIRROR>(v));
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<32>(v);
  return v + __shfl_xor(v, 32);
}

// Combine every lane with lane ^ 16 (or ^ 32) on the VALU: gfx950's
// permlane swaps hand each lane the pair {its own value, its partner's}, in
// either order, so a commutative operation over the pair gives both partners
// the same bits without a trip through the LDS crossbar.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ __forceinline__ int clamp_ctx(int c, int max_ctx) { return c < 0 ? 0 : (c > max_ctx ? max_ctx : c); }

// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
