// Split-partition paged decode on the gfx950 matrix cores (bf16 storage,
// fp32 accumulation).
//
// One work-group of kWaves waves per (sequence, KV head, partition).  The
// partition is cut into 32-token steps (mfma_step.h); wave w takes steps w,
// w + kWaves, ...  Loads run one step ahead of the math (two register sets).
// At the end the waves merge (m, l, O) through LDS; a single-partition
// sequence writes its normalised bf16 output directly, otherwise the partial
// goes to the workspace and decode_reduce.hip merges the partitions.
#include "mfma_step.h"

namespace pa {
namespace {

using namespace mfma;

// Waves per work-group, and the minimum waves per SIMD the register
// allocation must leave room for (tuning knobs; 0 = compiler's choice).
#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif
#ifndef PA_MFMA_MIN_WAVES_PER_EU
#define PA_MFMA_MIN_WAVES_PER_EU 0
#endif
constexpr int kWaves = PA_MFMA_WAVES;

template <int D>
__global__ __launch_bounds__(kWaves * 64)
#if PA_MFMA_MIN_WAVES_PER_EU > 0
__attribute__((amdgpu_waves_per_eu(PA_MFMA_MIN_WAVES_PER_EU)))
#endif
void decode_mfma_kernel(DecodeParams p) {
  constexpr int kKi = D / 32;
  __shared__ float sm_o[kWaves][16][D];
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];

  const WorkItem w = decode_work_item(p, blockIdx.x);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15;
  const int q4 = lane >> 4;
  const int G = p.group;
  const int len = p.seq_lens[w.seq];
  const int64_t out_row0 = (int64_t)w.seq * p.num_heads + (int64_t)w.head * G;
  uint16_t* out = (uint16_t*)p.out;

  if (!seq_len_ok(p, len) || len == 0) {
    if (w.part == 0) {
      const uint16_t fill = len == 0 ? (uint16_t)0 : (uint16_t)0x7FC0;
      for (int i = tid; i < G * D; i += kWaves * 64) out[out_row0 * D + i] = fill;
    }
    return;
  }
  const int pstart = w.part * p.partition_size;
  if (pstart >= len) return;
  const int pend = min(len, pstart + p.partition_size);
  const int nparts = ceil_div_i(len, p.partition_size);

  // Q^T as the B operand: column r16 = query head h*G + r16, zero when r16 >= G.
  u32x4 qb[kKi];
  {
    const char* qrow = (const char*)p.q + ((out_row0 + r16) * D) * 2 + q4 * 16;
#pragma unroll
    for (int i = 0; i < kKi; ++i)
      qb[i] = r16 < G ? *(const u32x4*)(qrow + 64 * i) : u32x4{0u, 0u, 0u, 0u};
  }

  SeqView c;
  const int64_t head_stride = (int64_t)p.block_size * D * 2;
  c.kbase = (const char*)p.k_cache + (int64_t)w.head * head_stride;
  c.vbase = (const char*)p.v_cache + (int64_t)w.head * head_stride;
  c.table = p.block_tables + (int64_t)w.seq * p.max_blocks_per_seq;
  c.block_stride = (int64_t)p.kv_heads * head_stride;
  c.nblocks_valid = (len + p.block_size - 1) >> p.block_shift;
  c.num_blocks = p.num_blocks;
  c.block_shift = p.block_shift;
  c.bmask = p.block_size - 1;

  Acc<D> a;
  reset(a);
  bool bad = false;

  // Two register sets, loads one step ahead of the math.
  const int stride = 32 * kWaves;
  int base = pstart + 32 * wave;
  if (base < pend) {
    StepRegs<D> ra, rb;
    load_step<D>(ra, c, base, r16, q4, bad);
    while (true) {
      int next = base + stride;
      if (next < pend) load_step<D>(rb, c, next, r16, q4, bad);
      compute_step<D>(ra, a, qb, base, pend, p.scale_log2, q4);
      base = next;
      if (base >= pend) break;
      next = base + stride;
      if (next < pend) load_step<D>(ra, c, next, r16, q4, bad);
      compute_step<D>(rb, a, qb, base, pend, p.scale_log2, q4);
      base = next;
      if (base >= pend) break;
    }
  }
  finish_wave(a, bad);
  stash_wave<D, kWaves>(a, sm_o, sm_m, sm_l, wave, r16, q4, G);
  __syncthreads();
  for (int i = tid; i < G * D; i += kWaves * 64) {
    const int g = i / D;
    const int d = i - g * D;
    float mx, l, o;
    merge_waves<D, kWaves>(sm_o, sm_m, sm_l, g, d, mx, l, o);
    if (nparts == 1) {
      out[(out_row0 + g) * D + d] = f32_to_bf16(o / l);
    } else {
      const int64_t slot = (out_row0 + g) * p.num_partitions + w.part;
      p.ws_o[slot * D + d] = o;
      if (d == 0) {
        p.ws_ml[slot * 2 + 0] = mx;
        p.ws_ml[slot * 2 + 1] = l;
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.num_partitions * p.num_seqs * p.kv_heads));
  const dim3 block(kWaves * 64);
  if (head_dim == 128)
    decode_mfma_kernel<128><<<grid, block, 0, stream>>>(p);
  else if (head_dim == 64)
    decode_mfma_kernel<64><<<grid, block, 0, stream>>>(p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
