// Matrix-core building blocks shared by the decode and prefill kernels: the
// 16x16x32 MFMA operand types, the online-softmax arithmetic of one wavefront
// over 32-token chunks, the transposed LDS reads of V, explicit memory-counter
// waits, and the LDS placement of 16-bit cache rows.
//
// Lane layouts of v_mfma_f32_16x16x32: lane l holds row l % 16 and the 8
// consecutive k-indices 8 * (l / 16) .. +7 of A; column l % 16 and the same
// k-indices of B; rows 4 * (l / 16) + i, i < 4, column l % 16 of C.  A chunk's
// scores are S^T = K q^T (tokens x columns) and the output update is
// O^T += V^T P^T, with the chunk's 32 tokens taken in the order
// tau(j, i) = 4 j + i (i < 4), 16 + 4 j + i - 4 (i >= 4), which makes each
// lane's 8 scores exactly its P^T operand.
#pragma once

#include "pa_device.h"

namespace pa {
namespace mfma {

constexpr int CT = 32;          // tokens per chunk: two 16-token QK tiles, one 32-token PV step
constexpr float kSlack = 8.0f;  // how far (log2 units) scores may exceed the running reference max

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) int32_t const_i32;

__device__ __forceinline__ const_i32 *as_const(const int32_t *p) { return (const_i32 *)(uintptr_t)p; }

// MFMA operand type (the query's 16-bit type)
template <typename MT> struct Op;
template <> struct Op<f16_t> {
  __device__ static f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
  __device__ static uint32_t bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
  __device__ static float value(uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); }
};
template <> struct Op<bf16_t> {
  __device__ static f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
  __device__ static uint32_t bits(float x) { return f32_to_bf16_rne(x); }
  __device__ static float value(uint32_t b) { return __builtin_bit_cast(float, b << 16); }
};

// Two ds_read_b64_tr_b16 (8 bytes at each lane's address, transposed across
// each 16-lane group) forming one 16x16x32 operand.
__device__ __forceinline__ u32x4 read_tr(const void *p0, const void *p1) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)p0);
  const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)p1);
  const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
  return u32x4{w0[0], w0[1], w1[0], w1[1]};
}

// The same read issued as inline assembly, for LDS filled by direct
// global-to-LDS loads: the compiler then adds no wait for the DMA stream (the
// caller's vmcnt waits order it), and the caller awaits completion with
// lgkm_wait on the destination registers.
__device__ __forceinline__ u32x2 tr_read_async(const char *p) {
  u32x2 d;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(d) : "v"((uint32_t)(uintptr_t)p));
  return d;
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x2 &x0, u32x2 &x1, u32x2 &x2, u32x2 &x3) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3) : "n"(N));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // vmcnt in bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8) left at their maxima
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <typename OT>
__device__ __forceinline__ void store4(void *base, int64_t off, const float *x) {
  if constexpr (__is_same(OT, f32_t)) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __builtin_bit_cast(uint32_t, x[i]);
    st16(reinterpret_cast<float *>(base) + off, w);
  } else {
    u32x2 w;
#pragma unroll
    for (int i = 0; i < 2; ++i) w[i] = Op<OT>::bits(x[2 * i]) | (Op<OT>::bits(x[2 * i + 1]) << 16);
    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(base) + off) = w;
  }
}

// LDS placement of 32 16-bit cache rows of D elements (one half-chunk slot):
// granule g (16 bytes) of row r sits at granule phys(r, g).  Granules are
// grouped in 256-byte lines and permuted inside a line by an XOR with a
// per-line constant, chosen so that the 16 rows of one K operand read fall
// on 16 different bank groups and the 8 rows that each half of a transposed
// V read covers fall on 8 different 32-byte bank groups.
template <int D>
struct RowSlot {
  static constexpr int RB = 2 * D;       // bytes per cache row
  static constexpr int GPR = RB / 16;    // 16-byte granules per row
  static constexpr int HB = CT * RB;     // bytes of a slot
  static constexpr int NLD = HB / 1024;  // wave-wide 16-byte DMA instructions per slot
  static constexpr int RPI = 1024 / RB;  // rows per DMA instruction
  static_assert(RPI <= 16 && 16 % RPI == 0, "a DMA instruction stays inside one 16-token tile");
  __device__ static __forceinline__ int swz(bool isv, int L) {
    return isv ? 2 * (L & (GPR / 2 - 1)) : (L & (GPR - 1));
  }
  __device__ static __forceinline__ int phys(bool isv, int r, int g) {
    const int q = r * GPR + g, L = q >> 4;
    return (L << 4) | ((q & 15) ^ swz(isv, L));
  }
  // the row and granule that lane `lane` of DMA instruction i brings into the slot
  __device__ static __forceinline__ void dma_target(bool isv, int i, int lane, int &r, int &g) {
    const int P = 64 * i + lane;  // LDS granule this lane fills
    const int L = P >> 4;
    const int q = (L << 4) | ((P & 15) ^ swz(isv, L));
    r = q / GPR;
    g = q % GPR;
  }
  // byte offset of lane (c16, j)'s K operand of k-step kb, tile 0
  __device__ static __forceinline__ int k_off(int c16, int j, int kb) { return 16 * phys(false, c16, 4 * kb + j); }
  // byte offset of lane (c16, j)'s first half of the V^T operand of output tile n
  __device__ static __forceinline__ int v_off(int c16, int j, int n) {
    return 16 * phys(true, 4 * j + (c16 >> 2), 2 * n + ((c16 & 3) >> 1)) + 8 * (c16 & 1);
  }
};

// The arithmetic of one wavefront over chunks of 32 tokens against the 16
// columns of its queries: scores, online softmax with a lazy rescale, output
// update.  Lane (c16, j) keeps the softmax state of column c16 (combined over
// the 4 quarters j by finish()) and the O^T tiles of dims 16 n + 4 j + i.
template <typename MT, int D>
struct MfmaCore {
  static constexpr int KS = D / 32;  // k-steps of the QK contraction
  static constexpr int NT = D / 16;  // 16-dim output tiles

  const int c16, j;  // column / row within 16, quarter of the wave
  float m, l;        // softmax state of column c16 (lane-local until finish())
  f32x4 acc[NT];

  __device__ explicit MfmaCore(int lane) : c16(lane & 15), j(lane >> 4) {}
  __device__ MfmaCore() : MfmaCore(__lane_id()) {}

  __device__ __forceinline__ void reset() {
    m = -INFINITY;
    l = 0.0f;
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // S^T of the chunk's two 16-token tiles; kop(tt, kb) is the A operand
  // K[16 tt + c16][32 kb + 8 j ..]
  template <class KOp>
  __device__ __forceinline__ void scores(const u32x4 *qop, KOp kop, f32x4 *sc) const {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sc[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < KS; ++kb) sc[tt] = Op<MT>::mma(kop(tt, kb), qop[kb], sc[tt]);
    }
  }

  // Online softmax for column c16 over the lane's 8 tokens of the chunk
  // starting at token cs (those past `last`, the column's last visible token,
  // masked), then across the 4 quarters; returns the weights as P^T operands
  // split as P = hi + lo in the operand type.  EMPTY_OK: the column may have
  // seen no position yet and see none in this chunk either (its running max
  // still -inf); its weights are then zeros instead of exp2(-inf - -inf).
  // TILE_SCALES: each 16-token tile tt has its own key factor kf[tt] (on its
  // scores) and value factor vf[tt] (on its weights in P, not in the sum l).
  template <bool EMPTY_OK = false, bool TILE_SCALES = false>
  __device__ __forceinline__ void weights(const f32x4 *sc, int cs, int last, float qk_scale_log2, u32x4 &phi,
                                          u32x4 &plo, const float *kf = nullptr, const float *vf = nullptr) {
    float p8[8];
    float cm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tok = (i < 4 ? 4 * j + i : 16 + 4 * j + i - 4);
      const float x = sc[i >> 2][i & 3] * (TILE_SCALES ? qk_scale_log2 * kf[i >> 2] : qk_scale_log2);
      p8[i] = cs + tok <= last ? x : -INFINITY;
      cm = fmaxf(cm, p8[i]);
    }
    cm = max_xor32(max_xor16(cm));
    // lazy rescale: the reference max moves only when a score exceeds it by
    // more than kSlack (log2 units), so weights stay below 2^kSlack and the
    // accumulator rescale is skipped for almost every chunk
    if (__ballot(cm > m + kSlack)) {
      const float mn = fmaxf(m, cm);
      // (a column that has seen nothing yet rescales its zeros by 0, never by exp2(NaN))
      const float alpha = EMPTY_OK && m == -INFINITY ? 0.0f : fast_exp2(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] *= alpha;
    }
    const float mn = EMPTY_OK && m == -INFINITY ? 0.0f : m;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      float e0 = fast_exp2(p8[i] - mn), e1 = fast_exp2(p8[i + 1] - mn);
      l += e0 + e1;
      if (TILE_SCALES) {  // tokens i and i + 1 share a tile
        e0 *= vf[i >> 2];
        e1 *= vf[i >> 2];
      }
      const uint32_t h0 = Op<MT>::bits(e0), h1 = Op<MT>::bits(e1);
      phi[i >> 1] = h0 | (h1 << 16);
      plo[i >> 1] = Op<MT>::bits(e0 - Op<MT>::value(h0)) | (Op<MT>::bits(e1 - Op<MT>::value(h1)) << 16);
    }
  }

  // O^T += V^T P^T; vop(n) is the A operand V[tau(j, i)][16 n + c16], i < 8
  template <class VOp>
  __device__ __forceinline__ void accumulate(u32x4 phi, u32x4 plo, VOp vop) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const u32x4 vt = vop(n);
      acc[n] = Op<MT>::mma(vt, phi, acc[n]);
      acc[n] = Op<MT>::mma(vt, plo, acc[n]);
    }
  }

  // accumulate() with the V^T operands read from a ring slot by the assembly
  // reads (see accumulate_slot_n)
  template <class VOff>
  __device__ __forceinline__ void accumulate_slot(u32x4 phi, u32x4 plo, const char *vs, VOff voff);

  __device__ __forceinline__ void finish() { l = sum_xor32(sum_xor16(l)); }
};

// O^T += V^T P^T for NC cores (16 columns each) that share the chunk's V rows:
// the V^T operands are read once from a ring slot by the assembly reads, two
// tiles of reads in flight ahead of the tiles being multiplied, and each
// operand is multiplied into every core; voff(n) is the lane's byte offset of
// tile n's first half.
template <int NC, typename MT, int D, class VOff>
__device__ __forceinline__ void accumulate_slot_n(MfmaCore<MT, D> *core, const u32x4 *phi, const u32x4 *plo,
                                                  const char *vs, VOff voff) {
  constexpr int NT = D / 16;
  constexpr int RB = 2 * D;
  u32x2 vt[NT][2];
#pragma unroll
  for (int n = 0; n < 4 && n < NT; ++n) {
    vt[n][0] = tr_read_async(vs + voff(n));
    vt[n][1] = tr_read_async(vs + voff(n) + 16 * RB);
  }
#pragma unroll
  for (int n = 0; n < NT; n += 2) {
    // reads issued after tiles n, n+1: those of tiles n+2, n+3, if any
    if (n + 3 < NT)
      lgkm_wait<4>(vt[n][0], vt[n][1], vt[n + 1][0], vt[n + 1][1]);
    else
      lgkm_wait<0>(vt[n][0], vt[n][1], vt[n + 1][0], vt[n + 1][1]);
    if (n + 4 < NT) {
      vt[n + 4][0] = tr_read_async(vs + voff(n + 4));
      vt[n + 4][1] = tr_read_async(vs + voff(n + 4) + 16 * RB);
      vt[n + 5][0] = tr_read_async(vs + voff(n + 5));
      vt[n + 5][1] = tr_read_async(vs + voff(n + 5) + 16 * RB);
    }
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const u32x4 op{vt[n + d][0][0], vt[n + d][0][1], vt[n + d][1][0], vt[n + d][1][1]};
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        core[ct].acc[n + d] = Op<MT>::mma(op, phi[ct], core[ct].acc[n + d]);
        core[ct].acc[n + d] = Op<MT>::mma(op, plo[ct], core[ct].acc[n + d]);
      }
    }
  }
}

template <typename MT, int D>
template <class VOff>
__device__ __forceinline__ void MfmaCore<MT, D>::accumulate_slot(u32x4 phi, u32x4 plo, const char *vs, VOff voff) {
  accumulate_slot_n<1>(this, &phi, &plo, vs, voff);
}

}  // namespace mfma
}  // namespace pa
