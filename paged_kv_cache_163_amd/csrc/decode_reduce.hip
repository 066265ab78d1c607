// Cross-partition merge for split-sequence decode.
//
// Partition p of a sequence left, per query head, its running max m_p (base-2
// units), running sum l_p = sum exp2(s - m_p) and unnormalised output
// o_p = sum exp2(s - m_p) v.  With M = max_p m_p and w_p = exp2(m_p - M):
//     out = (sum_p w_p o_p) / (sum_p w_p l_p),
// the same softmax-weighted average as one pass over the whole history.
//
// One 128-thread work-group per (sequence, query head); thread d owns output
// element d.  Up to kRegParts partitions, every thread loads all partitions'
// (m_p, l_p) (the same addresses for the whole work-group, so scalar loads)
// and its own o_p[d] in one round of loads and merges in registers: one
// memory latency and no barrier.  Longer lists compute the weights w_p once
// into LDS, then each thread sums its element over the partitions
// (consecutive threads read consecutive elements of o_p).
#include <math.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 128;
constexpr int kRegParts = 32;

__device__ inline float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = fmaxf(red[0], red[1]);
  __syncthreads();
  return v;
}

__device__ inline float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = red[0] + red[1];
  __syncthreads();
  return v;
}

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void decode_reduce_kernel(DecodeParams p) {
  extern __shared__ float sm_w[];  // [num_partitions] weights w_p
  __shared__ float red[2];
  const int hq = blockIdx.x % p.num_heads;
  const int seq = blockIdx.x / p.num_heads;
  const int len = p.seq_lens[seq];
  if (!seq_len_ok(p, len)) return;  // the partition kernel already wrote NaN
  const int nparts = ceil_div_i(len, p.partition_size);
  if (nparts <= 1) return;          // written directly by the partition kernel
  const int64_t slot0 = ((int64_t)seq * p.num_heads + hq) * p.num_partitions;
  const int64_t layer = blockIdx.y;  // layered pool: one grid row per decoded layer
  const float* ml = p.ws_ml + layer * (p.layer_ws_stride / D) * 2 + slot0 * 2;
  const float* o = p.ws_o + layer * p.layer_ws_stride + slot0 * D;
  const int d0 = threadIdx.x;
  if (nparts <= kRegParts) {
    if (d0 >= D) return;
    float mv[kRegParts], lv[kRegParts], ov[kRegParts];
#pragma unroll
    for (int q = 0; q < kRegParts; ++q) {
      if (q < nparts) {
        mv[q] = ml[2 * q];
        lv[q] = ml[2 * q + 1];
        ov[q] = o[(int64_t)q * D + d0];
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < kRegParts; ++q)
      if (q < nparts) mx = fmaxf(mx, mv[q]);
    float l = 0.f, acc = 0.f;
#pragma unroll
    for (int q = 0; q < kRegParts; ++q) {
      if (q < nparts) {
        const float w = exp2f(mv[q] - mx);
        l += w * lv[q];
        acc += w * ov[q];
      }
    }
    const float r = acc / l;
    const int64_t idx = layer * p.layer_q_stride + ((int64_t)seq * p.num_heads + hq) * D + d0;
    if (BF16)
      ((uint16_t*)p.out)[idx] = f32_to_bf16(r);
    else
      ((float*)p.out)[idx] = r;
    return;
  }

  float mx = -INFINITY;
  for (int q = threadIdx.x; q < nparts; q += kThreads) mx = fmaxf(mx, ml[2 * q]);
  mx = block_max(mx, red);
  float l = 0.f;
  for (int q = threadIdx.x; q < nparts; q += kThreads) {
    const float w = exp2f(ml[2 * q] - mx);
    sm_w[q] = w;
    l += w * ml[2 * q + 1];
  }
  l = block_sum(l, red);  // its barriers also publish sm_w
  const float inv = 1.0f / l;
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float acc = 0.f;
    for (int q = 0; q < nparts; ++q) acc += sm_w[q] * o[(int64_t)q * D + d];
    const float r = acc * inv;
    const int64_t idx = layer * p.layer_q_stride + ((int64_t)seq * p.num_heads + hq) * D + d;
    if (BF16)
      ((uint16_t*)p.out)[idx] = f32_to_bf16(r);
    else
      ((float*)p.out)[idx] = r;
  }
}

template <bool BF16, int D>
hipError_t launch(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.num_seqs * p.num_heads),
                  (unsigned)(p.num_layers > 1 ? p.num_layers : 1));
  const size_t lds = (size_t)p.num_partitions * sizeof(float);
  decode_reduce_kernel<BF16, D><<<grid, kThreads, lds, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeParams& p, bool is_bf16, int head_dim,
                                hipStream_t stream) {
  if ((size_t)p.num_partitions * sizeof(float) > 64 * 1024) return hipErrorInvalidValue;
  if (is_bf16) {
    if (head_dim == 64) return launch<true, 64>(p, stream);
    if (head_dim == 128) return launch<true, 128>(p, stream);
  } else {
    if (head_dim == 64) return launch<false, 64>(p, stream);
    if (head_dim == 128) return launch<false, 128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
