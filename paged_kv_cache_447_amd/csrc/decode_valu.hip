// Paged decode, split-context partition kernel, vector-ALU path.
//
// One workgroup (4 wave64s) per (context partition, kv head, sequence).  The
// table lookup follows the logical-to-physical translation of the page
// "vLLM框架中的KV cache优化与PagedAttention机制详解" (section 5.1: find the KV range,
// map logical block numbers to physical ones, handle reads that cross blocks),
// with the address rule physical = block * block_size + offset of page
// "Paged KVCache：大模型推理显存管理优化方案" (section 2.3).  The per-block score /
// cross-block accumulation split is the one page
// "vLLM推理引擎架构：PagedAttention机制与高吞吐推理" (section 2.3) describes.
//
// Data movement (the whole cost of this kernel):
//   A token's K row for one kv head is head_dim * elem bytes, contiguous.  LPR
//   lanes cover it with 16-byte loads, so one wave-wide load instruction reads
//   TPW = 64 / LPR consecutive tokens of one block.  A wave takes chunks of
//   CH = TPW * NL tokens (chunks of a partition are dealt round-robin to the 4
//   waves), issuing all NL K loads and NL V loads of a chunk before using any,
//   so 2 * NL * 1 KiB per wave are in flight.  The block id of each load is
//   wave-uniform and comes through the scalar cache.
//
// Arithmetic per chunk (fp32): score = (q * scale * log2 e) . K via per-lane
// FMAs and a DPP sum over the LPR lanes of a token; a running max m and sum l
// per wave with the usual rescale by exp2(m_old - m_new); acc += p * V.  Waves
// merge their (m, l, acc) through LDS at the end.  A partition that is its
// sequence's only one writes the normalised output; otherwise it writes
// (m, l, acc) to the workspace for the log-sum-exp merge kernel.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <typename QT>
__device__ __forceinline__ void store_out(const DecodeArgs &a, int64_t idx, float x) {
  if (a.out_f32)
    reinterpret_cast<float *>(a.out)[idx] = x;
  else
    Elem<QT>::store(a.out, idx, x);
}

template <typename KVT, typename QT, int D, int G, int NL>
__global__ void __launch_bounds__(kThreads) decode_partition_valu(const DecodeArgs a) {
  constexpr int VEC = Elem<KVT>::kPer16;  // KV elements per 16-byte load
  constexpr int LPR = D / VEC;            // lanes per token row
  constexpr int TPW = 64 / LPR;           // tokens per wave-wide load
  constexpr int CH = TPW * NL;            // tokens per wave chunk
  static_assert(LPR >= 4 && LPR <= 32, "row must span 4..32 lanes");

  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  __shared__ float sm_acc[kWaves][G][D];

  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  int ctx = a.context_lens[seq];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int t0 = part * a.partition_size;
  if (t0 >= ctx) {
    if (part == 0) {  // empty context: the output is zero
      for (int i = threadIdx.x; i < G * D; i += kThreads) {
        const int h = kvh * G + i / D;
        store_out<QT>(a, (int64_t)seq * a.o_ss + (int64_t)h * a.o_sh + i % D, 0.0f);
      }
    }
    return;
  }
  const int t1 = min(ctx, t0 + a.partition_size);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane % LPR;  // which 16-byte slice of the row
  const int g = lane / LPR;  // which token of a wave-wide load

  // query slice, pre-scaled into the log2 domain
  float qf[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int64_t base = (int64_t)seq * a.q_ss + (int64_t)(kvh * G + h) * a.q_sh + r * VEC;
#pragma unroll
    for (int v = 0; v < VEC; ++v) qf[h][v] = Elem<QT>::load(a.q, base + v) * a.qk_scale_log2;
  }

  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[h][v] = 0.0f;
  }

  const int32_t *bt = a.block_tables + (int64_t)seq * a.bt_ss;
  const char *kb = reinterpret_cast<const char *>(a.k_cache) +
                   ((int64_t)kvh * a.k_sh + r * VEC) * Elem<KVT>::kBytes;
  const char *vb = reinterpret_cast<const char *>(a.v_cache) +
                   ((int64_t)kvh * a.v_sh + r * VEC) * Elem<KVT>::kBytes;
  const int bmask = a.block_size - 1;
  const int nchunks = (t1 - t0 + CH - 1) / CH;

  for (int c = wave; c < nchunks; c += kWaves) {
    const int cb = t0 + c * CH;
    u32x4 kr[NL], vr[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int tu = cb + i * TPW;  // wave-uniform first token of this load
      if (tu < t1) {
        int blk = bt[tu >> a.log2_block_size];
        blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
        const int tok = (tu & bmask) + g;
        kr[i] = ld16(kb + ((int64_t)blk * a.k_sb + (int64_t)tok * a.k_st) * Elem<KVT>::kBytes);
        vr[i] = ld16(vb + ((int64_t)blk * a.v_sb + (int64_t)tok * a.v_st) * Elem<KVT>::kBytes);
      } else {
        kr[i] = u32x4{0u, 0u, 0u, 0u};
        vr[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }

    float s[G][NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float kf[VEC];
      Elem<KVT>::unpack(kr[i], kf);
      const bool valid = cb + i * TPW + g < t1;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.0f;
#pragma unroll
        for (int v = 0; v < VEC; ++v) d = __builtin_fmaf(qf[h][v], kf[v], d);
        d = group_sum<LPR>(d);
        s[h][i] = valid ? d : -INFINITY;
      }
      // masked rows may hold anything (NaN included): keep them out of p * V
      if (!valid) vr[i] = u32x4{0u, 0u, 0u, 0u};
    }

#pragma unroll
    for (int h = 0; h < G; ++h) {
      float cm = s[h][0];
#pragma unroll
      for (int i = 1; i < NL; ++i) cm = fmaxf(cm, s[h][i]);
      cm = across_groups_max<LPR>(cm);
      const float mn = fmaxf(m[h], cm);
      const float alpha = fast_exp2(m[h] - mn);
      l[h] *= alpha;
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[h][v] *= alpha;
#pragma unroll
      for (int i = 0; i < NL; ++i) s[h][i] = fast_exp2(s[h][i] - mn);
      m[h] = mn;
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float vf[VEC];
      Elem<KVT>::unpack(vr[i], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        l[h] += s[h][i];
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[h][v] = __builtin_fmaf(s[h][i], vf[v], acc[h][v]);
      }
    }
  }

  // combine the TPW token groups of the wave, then the waves through LDS
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = across_groups_sum<LPR>(l[h]);
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[h][v] = across_groups_sum<LPR>(acc[h][v]);
  }
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int v = 0; v < VEC; ++v) sm_acc[wave][h][r * VEC + v] = acc[h][v];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm_m[wave][h] = m[h];
      sm_l[wave][h] = l[h];
    }
  }
  __syncthreads();

  const bool single = ctx <= a.partition_size;
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    float M = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = fast_exp2(sm_m[w][h] - M);
      L = __builtin_fmaf(e, sm_l[w][h], L);
      O = __builtin_fmaf(e, sm_acc[w][h][d], O);
    }
    const int head = kvh * G + h;
    if (single) {
      store_out<QT>(a, (int64_t)seq * a.o_ss + (int64_t)head * a.o_sh + d, O / L * a.v_scale);
    } else {
      const int64_t row = ((int64_t)seq * a.num_heads + head) * a.num_partitions + part;
      a.ws_acc[row * D + d] = O;
      if (d == 0) {
        a.ws_ml[row * 2] = M;
        a.ws_ml[row * 2 + 1] = L;
      }
    }
  }
}

template <typename KVT, typename QT, int D, int G>
hipError_t launch_one(const DecodeArgs &a, hipStream_t stream) {
  constexpr int NL = 8;
  dim3 grid(a.num_partitions, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_partition_valu<KVT, QT, D, G, NL>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename KVT, typename QT, int D>
hipError_t dispatch_group(const DecodeArgs &a, hipStream_t stream) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return launch_one<KVT, QT, D, 1>(a, stream);
    case 2: return launch_one<KVT, QT, D, 2>(a, stream);
    case 4: return launch_one<KVT, QT, D, 4>(a, stream);
    case 8: return launch_one<KVT, QT, D, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename KVT, typename QT>
hipError_t dispatch_dim(const DecodeArgs &a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return dispatch_group<KVT, QT, 64>(a, stream);
    case 128: return dispatch_group<KVT, QT, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_supported(int kv_kind, int q_kind, int head_dim, int group) {
  const bool pair = (kv_kind == q_kind && kv_kind != KV_FP8) ||
                    (kv_kind == KV_FP8 && (q_kind == KV_F16 || q_kind == KV_BF16));
  return pair && (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_decode_partitions(const DecodeArgs &a, hipStream_t stream) {
  switch (a.kv_kind) {
    case KV_F32: return dispatch_dim<f32_t, f32_t>(a, stream);
    case KV_F16: return dispatch_dim<f16_t, f16_t>(a, stream);
    case KV_BF16: return dispatch_dim<bf16_t, bf16_t>(a, stream);
    case KV_FP8:
      if (a.q_kind == KV_F16) return dispatch_dim<fp8_t, f16_t>(a, stream);
      if (a.q_kind == KV_BF16) return dispatch_dim<fp8_t, bf16_t>(a, stream);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
