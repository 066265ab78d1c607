// Cross-partition merge for split-sequence decode.
//
// Partition p of a sequence left, per query head, its running max m_p (base-2
// units), running sum l_p = sum exp2(s - m_p) and unnormalised output
// o_p = sum exp2(s - m_p) v.  With M = max_p m_p and w_p = exp2(m_p - M):
//     out = (sum_p w_p o_p) / (sum_p w_p l_p),
// the same softmax-weighted average as one pass over the whole history.
//
// One 128-thread work-group per (sequence, query head): the weights w_p are
// computed once into LDS, then each thread sums one head-dim element over the
// partitions (consecutive threads read consecutive elements of o_p).
#include <math.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 128;

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
  const float* o = p.ws_o + layer * p.layer_ws_stride + slot0 * D;
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

// Shared-prefix decode: each row's prefix partials (slots [0, kp), one per
// prefix partition) and tail partials (slots prefix.parts + [0, tp)) merge
// with the same weights as above.  One 256-thread work-group per (sequence,
// KV head): wave w computes the weights of query heads w, w + 4, ... into
// LDS, then the threads sum one output element each.  A member whose table
// does not start with its leader's prefix blocks, or whose length stops
// inside the prefix, gets a NaN row (the prefix partials were not its keys).
constexpr int kMergeThreads = 256;

__device__ inline float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ inline float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int D>
__global__ __launch_bounds__(kMergeThreads) void prefix_merge_kernel(DecodeParams p) {
  extern __shared__ float sm_pw[];  // [G][n] weights w_q
  __shared__ float sm_inv[16];
  __shared__ int sm_bad;
  const int head = blockIdx.x % p.kv_heads;
  const int seq = blockIdx.x / p.kv_heads;
  const int len = p.seq_lens[seq];
  if (!seq_len_ok(p, len)) return;  // the tail kernel already wrote NaN
  const int grp = shared_prefix_group(p.prefix, seq);
  const int pfx = grp >= 0 ? p.prefix.tokens[grp] : 0;
  const int kp = pfx > 0 ? ceil_div_i(pfx, p.prefix.partition) : 0;
  const int tp = len > pfx ? ceil_div_i(len - pfx, p.partition_size) : 0;
  if (pfx == 0 && tp <= 1) return;  // the tail kernel wrote the row itself
  const int G = p.group;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (tid == 0) sm_bad = pfx > 0 && len < pfx;
  __syncthreads();
  if (pfx > 0) {
    const int32_t* mine = p.block_tables + (int64_t)seq * p.max_blocks_per_seq;
    const int32_t* lead = p.block_tables + (int64_t)p.prefix.start[grp] * p.max_blocks_per_seq;
    bool diff = false;
    for (int j = tid; j < (pfx >> p.block_shift); j += kMergeThreads) diff |= mine[j] != lead[j];
    if (diff) sm_bad = 1;  // every writer stores the same value
  }
  const int n = kp + tp;
  const int64_t row0 = (int64_t)seq * p.num_heads + (int64_t)head * G;
  for (int g = wave; g < G; g += kMergeThreads / 64) {
    const float* ml = p.ws_ml + (row0 + g) * p.num_partitions * 2;
    float mx = -INFINITY;
    for (int i = lane; i < n; i += 64) {
      const int slot = i < kp ? i : p.prefix.parts + (i - kp);
      mx = fmaxf(mx, ml[2 * slot]);
    }
    mx = wave_max(mx);
    float l = 0.f;
    for (int i = lane; i < n; i += 64) {
      const int slot = i < kp ? i : p.prefix.parts + (i - kp);
      const float w = exp2f(ml[2 * slot] - mx);
      sm_pw[g * n + i] = w;
      l += w * ml[2 * slot + 1];
    }
    l = wave_sum(l);
    if (lane == 0) sm_inv[g] = 1.0f / l;
  }
  __syncthreads();
  const bool bad = sm_bad != 0;
  uint16_t* out = (uint16_t*)p.out;
  for (int i = tid; i < G * D; i += kMergeThreads) {
    const int g = i / D;
    const int d = i - g * D;
    const float* o = p.ws_o + (row0 + g) * p.num_partitions * D + d;
    float acc = 0.f;
    for (int q = 0; q < n; ++q) {
      const int slot = q < kp ? q : p.prefix.parts + (q - kp);
      acc += sm_pw[g * n + q] * o[(int64_t)slot * D];
    }
    out[(row0 + g) * D + d] = bad ? (uint16_t)0x7FC0 : f32_to_bf16(acc * sm_inv[g]);
  }
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

hipError_t launch_prefix_merge(const DecodeParams& p, int head_dim, hipStream_t stream) {
  const size_t lds = (size_t)p.group * p.num_partitions * sizeof(float);
  if (lds > 64 * 1024 || p.group > 16) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((int64_t)p.num_seqs * p.kv_heads));
  if (head_dim == 64)
    prefix_merge_kernel<64><<<grid, kMergeThreads, lds, stream>>>(p);
  else if (head_dim == 128)
    prefix_merge_kernel<128><<<grid, kMergeThreads, lds, stream>>>(p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
