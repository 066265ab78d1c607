// Cross-partition merge for split-sequence decode.
//
// Partition p of a sequence left, per query head, its running max m_p (base-2
// units), running sum l_p = sum exp2(s - m_p) and unnormalised output
// o_p = sum exp2(s - m_p) v.  With M = max_p m_p and w_p = exp2(m_p - M):
//     out = (sum_p w_p o_p) / (sum_p w_p l_p),
// the same softmax-weighted average as one pass over the whole history.
// One work-group per (sequence, KV head) covers the G query heads of the
// group; consecutive threads take consecutive head-dim elements.
#include <math.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void decode_reduce_kernel(DecodeParams p) {
  const int head = blockIdx.x % p.kv_heads;
  const int seq = blockIdx.x / p.kv_heads;
  const int len = p.seq_lens[seq];
  if (!seq_len_ok(p, len)) return;  // the partition kernel already wrote NaN
  const int nparts = ceil_div_i(len, p.partition_size);
  if (nparts <= 1) return;          // written directly by the partition kernel
  const int G = p.group;
  const int64_t row0 = (int64_t)seq * p.num_heads + (int64_t)head * G;
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int g = i / D;
    const int d = i - g * D;
    const int64_t slot0 = (row0 + g) * p.num_partitions;
    const float* ml = p.ws_ml + slot0 * 2;
    float mx = -INFINITY;
    for (int q = 0; q < nparts; ++q) mx = fmaxf(mx, ml[2 * q]);
    float o = 0.f, l = 0.f;
    for (int q = 0; q < nparts; ++q) {
      const float wt = exp2f(ml[2 * q] - mx);
      o += wt * p.ws_o[(slot0 + q) * D + d];
      l += wt * ml[2 * q + 1];
    }
    const float r = o / l;
    if (BF16)
      ((uint16_t*)p.out)[(row0 + g) * D + d] = f32_to_bf16(r);
    else
      ((float*)p.out)[(row0 + g) * D + d] = r;
  }
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeParams& p, bool is_bf16, int head_dim,
                                hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.num_seqs * p.kv_heads));
  if (is_bf16) {
    if (head_dim == 64) decode_reduce_kernel<true, 64><<<grid, kThreads, 0, stream>>>(p);
    else if (head_dim == 128) decode_reduce_kernel<true, 128><<<grid, kThreads, 0, stream>>>(p);
    else return hipErrorInvalidValue;
  } else {
    if (head_dim == 64) decode_reduce_kernel<false, 64><<<grid, kThreads, 0, stream>>>(p);
    else if (head_dim == 128) decode_reduce_kernel<false, 128><<<grid, kThreads, 0, stream>>>(p);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
