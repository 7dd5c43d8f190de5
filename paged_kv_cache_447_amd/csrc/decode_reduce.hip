// Log-sum-exp merge of split-context partitions.
//
// For a sequence longer than one partition, partition p left a running max m_p
// (log2 units), a sum l_p = sum exp2(s - m_p) and an unnormalised output
// acc_p = sum exp2(s - m_p) v.  With M = max_p m_p the exact result is
//   out = sum_p exp2(m_p - M) acc_p / sum_p exp2(m_p - M) l_p,
// i.e. the same softmax over the whole context, only summed in another order.
// One wave64 per (query head, sequence); each lane owns head_dim / 64 output
// elements; partition weights are staged in LDS once per workgroup.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kMaxStaged = 1024;  // partitions whose weights fit the LDS stage

template <typename QT>
__global__ void __launch_bounds__(64) decode_reduce_kernel(const DecodeArgs a) {
  __shared__ float sm_w[kMaxStaged];
  const int head = blockIdx.x;
  const int seq = blockIdx.y;
  int ctx = a.context_lens[seq];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  if (ctx <= a.partition_size) return;  // the partition kernel wrote the output itself
  const int np = (ctx + a.partition_size - 1) / a.partition_size;
  const int64_t row0 = ((int64_t)seq * a.num_heads + head) * a.num_partitions;
  const float *ml = a.ws_ml + row0 * 2;

  float M = -INFINITY;
  for (int p = threadIdx.x; p < np; p += 64) M = fmaxf(M, ml[2 * p]);
  M = wave_max(M);

  float L = 0.0f;
  for (int p = threadIdx.x; p < np; p += 64) {
    const float w = fast_exp2(ml[2 * p] - M);
    if (p < kMaxStaged) sm_w[p] = w;
    L = __builtin_fmaf(w, ml[2 * p + 1], L);
  }
  L = wave_sum(L);
  __syncthreads();

  const float inv = a.v_scale / L;
  const int64_t obase = (int64_t)seq * a.o_ss + (int64_t)head * a.o_sh;
  for (int d = threadIdx.x; d < a.head_dim; d += 64) {
    float O = 0.0f;
    for (int p = 0; p < np; ++p) {
      const float w = p < kMaxStaged ? sm_w[p] : fast_exp2(ml[2 * p] - M);
      O = __builtin_fmaf(w, a.ws_acc[(row0 + p) * a.head_dim + d], O);
    }
    const float x = O * inv;
    if (a.out_f32)
      reinterpret_cast<float *>(a.out)[obase + d] = x;
    else
      Elem<QT>::store(a.out, obase + d, x);
  }
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeArgs &a, hipStream_t stream) {
  dim3 grid(a.num_heads, a.num_seqs);
  switch (a.q_kind) {
    case KV_F32: hipLaunchKernelGGL(decode_reduce_kernel<f32_t>, grid, dim3(64), 0, stream, a); break;
    case KV_F16: hipLaunchKernelGGL(decode_reduce_kernel<f16_t>, grid, dim3(64), 0, stream, a); break;
    case KV_BF16: hipLaunchKernelGGL(decode_reduce_kernel<bf16_t>, grid, dim3(64), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
