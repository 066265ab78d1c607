// Chunked paged prefill on the gfx950 matrix cores (bf16 storage, fp32
// accumulation).
//
// Each sequence brings a chunk of queries whose keys and values are already
// in the cache: the last n of its L cached positions (a whole prompt when
// n = L).  The query at position p attends positions [0, p] through the
// sequence's block table (lihaoran.work PagedAttention explainer, section "A
// block table maps logical order to physical storage": causal attention over
// the visible history; logical block t / block_size, slot t % block_size).
//
// Rows are (chunk query, query head) pairs of one KV head's GQA group: row r
// of a work-group is query i0 + r / G, head g = r % G, so the G heads that
// share a KV head share every K/V load.  A work-group of kPfWaves waves covers
// kPrefillRows rows; each wave owns kRowTiles 16-row column tiles of the MFMA
// step from mfma_step.h (S^T = K Q^T, O^T += V^T P^T) with its Q^T operands in
// registers.  The work-group walks the keys [0, last position of its rows]
// in 32-token steps, staged straight from HBM into four LDS buffers three
// steps ahead of the math (row_tiles.h), so each K/V byte is fetched once per
// work-group.  A wave whose rows end earlier skips the math of the later
// steps.  The causal limit is per lane (a lane's score column is one row); V
// rows past the wave's last key are zeroed so tail slots never reach the
// sum.  The first step holds key 0, which every row sees, so no row's
// running max stays -inf after it.
//
// Work order: work-group x runs on XCD x % 8.  All query tiles of one
// (sequence, KV head) pair are given consecutive slots on one XCD, latest
// tile (most keys) first, so the pair's K/V stays in that XCD's L2 while its
// tiles run.
#include "row_tiles.h"

namespace pa {
namespace {

using namespace mfma;

template <int D>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_mfma_kernel(PrefillParams p) {
  constexpr int kVd = D / 16;
  const int pairs = p.num_seqs * p.kv_heads;
  const int x = blockIdx.x;
  const int slot = x >> 3;
  const int pair = (slot / p.q_tiles) * 8 + (x & 7);
  if (pair >= pairs) return;
  const int tile = p.q_tiles - 1 - (slot % p.q_tiles);
  const int seq = pair / p.kv_heads;
  const int head = pair - seq * p.kv_heads;
  const int q0 = p.query_start[seq];
  const int q1 = p.query_start[seq + 1];
  if (q0 < 0 || q1 > p.num_queries || q1 <= q0) return;  // no chunk, or offsets out of range
  const int nq = q1 - q0;
  const int len = p.seq_lens[seq];
  const int G = p.group;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15;
  const int q4 = lane >> 4;
  uint16_t* out = (uint16_t*)p.out;
  const int64_t row_stride = (int64_t)p.num_heads * D;  // elements per query
  const int64_t head0 = (int64_t)head * G * D;

  // A chunk the launch cannot serve (longer than its sequence or than the
  // host's bound, or a sequence past the table) gets NaN in every row of
  // this head group, written by tile 0; no cache or table read happens.
  const bool servable = nq <= len && nq <= p.max_query_len &&
                        (int64_t)len <= (int64_t)p.max_blocks_per_seq * p.block_size;
  if (!servable) {
    if (tile != 0) return;
    for (int64_t i = tid; i < (int64_t)nq * G * D; i += kPfWaves * 64) {
      const int64_t qi = i / (G * D);
      out[(q0 + qi) * row_stride + head0 + (i - qi * G * D)] = 0x7FC0;
    }
    return;
  }
  const int i0 = tile * (kPrefillRows / G);  // first chunk query of the work-group
  if (i0 >= nq) return;                       // the whole work-group: past the chunk
  const int pos0 = len - nq;                  // position of chunk query 0
  const int kend_wg = pos0 + min(nq - 1, i0 + (kPrefillRows - 1) / G) + 1;
  const int wrow0 = wave * kWaveRows;
  const int wi_first = i0 + wrow0 / G;
  const bool wave_rows = wi_first < nq;       // a wave past the chunk still stages tiles
  const int kend = wave_rows ? pos0 + min(nq - 1, i0 + (wrow0 + kWaveRows - 1) / G) + 1 : 0;
  // Last key every row of the wave sees (rows past the chunk have zero
  // queries and are never written, so unmasked steps may show them any key
  // below kend).
  const int kfull = pos0 + wi_first;

  SeqView c;
  const int64_t head_stride = (int64_t)p.block_size * D * 2;
  c.kbase = (const char*)p.k_cache + (int64_t)head * head_stride;
  c.vbase = (const char*)p.v_cache + (int64_t)head * head_stride;
  c.table = p.block_tables + (int64_t)seq * p.max_blocks_per_seq;
  c.block_stride = (int64_t)p.kv_heads * head_stride;
  c.nblocks_valid = (len + p.block_size - 1) >> p.block_shift;
  c.num_blocks = p.num_blocks;
  c.block_shift = p.block_shift;
  c.bmask = p.block_size - 1;

  PfAcc<D> a[kRowTiles];
#pragma unroll
  for (int nr = 0; nr < kRowTiles; ++nr) {
#pragma unroll
    for (int jt = 0; jt < kVd; ++jt) a[nr].o[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
    a[nr].l = f32x4{0.f, 0.f, 0.f, 0.f};
    a[nr].m = -INFINITY;
    a[nr].thr = -INFINITY;
  }
  bool bad = false;
  // Q^T operands of the lane's row in each tile (zero past the chunk) and the
  // causal limit of that row, loaded while the first key tiles are in flight.
  u32x4 qb[kRowTiles][D / 32];
  int lim[kRowTiles];
  auto load_q = [&] {
#pragma unroll
    for (int nr = 0; nr < kRowTiles; ++nr) {
      const int row = wrow0 + 16 * nr + r16;
      const int qi = i0 + row / G;
      const int g = row - (row / G) * G;
      const bool valid = qi < nq;
      lim[nr] = valid ? pos0 + qi : 0;
      const char* qrow = (const char*)p.q +
                         ((int64_t)(q0 + qi) * row_stride + head0 + (int64_t)g * D) * 2 + q4 * 16;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
        qb[nr][i] = valid ? *(const u32x4*)(qrow + 64 * i) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  __shared__ __attribute__((aligned(1024))) unsigned char sm_b[kLdsBufs][kStepBytes<D>];
  attend_keys<D>(a, c, qb, lim, 0, kend_wg, kend, len, kfull, wave_rows, p.scale_log2, bad, sm_b, wave,
                 lane, load_q);
  __syncthreads();   // every wave is done reading the buffers the output staging reuses
  if (!wave_rows) return;

  // The output rows go through LDS (wave w uses staging buffer w, free after
  // the barrier above; no staging is in flight): each wave writes its 32
  // normalised bf16 rows there and stores them back in whole 16-byte parts,
  // so every store instruction writes full rows (contiguous for the G heads
  // of one query) instead of a 32-byte piece of 16 rows.  A wave reads only
  // its own rows, and one wave's LDS operations complete in order.  Part k
  // of staged row r sits at slot k ^ swz(r), which makes the 16-byte reads
  // conflict-free (measured; a padded row stride leaves them 2-way).
  constexpr int kOutStride = D * 2;            // bytes per staged row
  constexpr int kParts = D * 2 / 16;           // 16-byte parts per row
  constexpr int kRowsPerStore = 64 / kParts;   // rows one store instruction covers
  static_assert(kWaveRows * kOutStride <= kStepBytes<D>, "fits");
  static_assert(kParts == 16 || kParts == 8, "row swizzle");
  auto swz = [](int r) { return kParts == 16 ? r & 15 : (r >> 1) & 7; };
  unsigned char* ow = sm_b[wave];
#pragma unroll
  for (int nr = 0; nr < kRowTiles; ++nr) {
    const float inv = bad ? __builtin_nanf("") : 1.0f / a[nr].l[0];
    // o[jt][rr] is head dim 16 jt + 4 q4 + rr of the lane's row: part
    // 2 jt + q4 / 2, byte 8 (q4 % 2) of it
    const int lr = 16 * nr + r16;
    unsigned char* lrow = ow + lr * kOutStride + 8 * (q4 & 1);
#pragma unroll
    for (int jt = 0; jt < kVd; ++jt) {
      const f32x4 o = a[nr].o[jt];
      *(u32x2*)(lrow + 16 * ((2 * jt + (q4 >> 1)) ^ swz(lr))) =
          u32x2{pack_bf16(o[0] * inv, o[1] * inv), pack_bf16(o[2] * inv, o[3] * inv)};
    }
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int it = 0; it < kWaveRows / kRowsPerStore; ++it) {
    const int lr = it * kRowsPerStore + lane / kParts;  // the wave's row 16 nr + r16
    const int part = lane % kParts;
    const int row = wrow0 + lr;
    const int qi = i0 + row / G;
    const int g = row - (row / G) * G;
    const u32x4 v = *(const u32x4*)(ow + lr * kOutStride + 16 * (part ^ swz(lr)));
    if (qi < nq)
      *(u32x4*)(out + (int64_t)(q0 + qi) * row_stride + head0 + (int64_t)g * D + 8 * part) = v;
  }
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillParams& p, int head_dim, hipStream_t stream) {
  const int64_t pairs8 = ((int64_t)p.num_seqs * p.kv_heads + 7) / 8 * 8;
  const dim3 grid((unsigned)(pairs8 * p.q_tiles));
  const dim3 block(kPfWaves * 64);
  if (head_dim == 128)
    prefill_mfma_kernel<128><<<grid, block, 0, stream>>>(p);
  else if (head_dim == 64)
    prefill_mfma_kernel<64><<<grid, block, 0, stream>>>(p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
