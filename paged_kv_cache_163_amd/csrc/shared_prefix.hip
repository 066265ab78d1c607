// Shared-prefix decode: groups of sequences whose block tables start with the
// same physical blocks (one prefix, refcounted, N tables pointing at it: "How
// PagedAttention works", section "A strong answer"; lihaoran.work explainer,
// section "Shared prefixes need matching computation").
//
// Plain decode reads a shared prefix block once per sequence.  Here the
// decode queries of all members of a group attend the shared keys together:
// rows are (member, query head) pairs of one KV head, 128 per work-group, over
// one partition of the prefix keys, on the row-tile engine of row_tiles.h, so
// each shared K/V tile is fetched once per work-group and the contraction runs
// on the matrix cores at 128 rows instead of G.  No causal limit applies: a
// decode query sits after its whole prefix.  Each member's positions after the
// prefix go through the decode work-group (decode_mfma.h, tail mode).  Both
// leave softmax partials (unnormalised O, max m, sum l) in the workspace, and
// prefix_merge_kernel combines them with the cross-partition formula of
// decode_reduce.hip.
//
// The prefix and tail work-groups share one launch, prefix first.  The host
// splits the prefix keys so that the prefix work-groups take about one of the
// two work-group slots of each compute unit; they run longest, and the short,
// latency-bound tail work-groups stream through the other slot meanwhile
// (measured on the shared-prefix workload: 78 us for the call against 94 us
// with the prefix and the tails in two launches, and 98 us with the two kinds
// alternating in one launch; the layouts were compared on one box in one
// run).
#include "decode_mfma.h"
#include "row_tiles.h"

namespace pa {
namespace {

using namespace mfma;

// Prefix part: work-group x of the prefix attention.  Group g owns prefix
// work-groups wg_start[g] ..; inside it, all member tiles of one (partition,
// KV head) pair run on one XCD (x % 8 is kept from the launch index), so the
// pair's K/V tiles stay in that XCD's L2.
template <int D>
__device__ __forceinline__ void prefix_wg(const DecodeParams& p, int x,
                                          unsigned char (*buf)[kStepBytes<D>]) {
  constexpr int kVd = D / 16;
  const PrefixGroups& pg = p.prefix;
  int grp = 0;
  for (int i = 1; i < pg.num_groups; ++i)
    if (x >= pg.wg_start[i]) grp = i;
  const int local = x - pg.wg_start[grp];
  const int first = pg.start[grp];
  const int members = pg.start[grp + 1] - first;
  const int tokens = pg.tokens[grp];
  const int G = p.group;
  const int tiles = ceil_div_i(members * G, kPrefillRows);
  const int combos = p.kv_heads * ceil_div_i(tokens, pg.partition);
  const int slot = local >> 3;
  const int combo = (slot / tiles) * 8 + (local & 7);
  if (combo >= combos) return;
  const int tile = slot - (slot / tiles) * tiles;
  const int head = combo % p.kv_heads;
  const int kp = combo / p.kv_heads;
  const int kstart = kp * pg.partition;
  const int kend_wg = range_end(kstart, pg.partition, tokens);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15;
  const int q4 = lane >> 4;
  const int m0 = tile * (kPrefillRows / G);  // first member of the work-group
  const int wrow0 = wave * kWaveRows;
  const bool wave_rows = m0 + wrow0 / G < members;
  // every row sees every key of the partition: the mask only cuts the last
  // step at kend_wg
  const int kend = wave_rows ? kend_wg : kstart;
  const int kfull = kend_wg - 1;

  SeqView c;
  const int64_t head_stride = (int64_t)p.block_size * D * 2;
  c.kbase = (const char*)p.k_cache + (int64_t)head * head_stride;
  c.vbase = (const char*)p.v_cache + (int64_t)head * head_stride;
  c.table = p.block_tables + (int64_t)first * p.max_blocks_per_seq;  // the leader's row
  c.block_stride = (int64_t)p.kv_heads * head_stride;
  c.nblocks_valid = tokens >> p.block_shift;
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
  // Q^T operands of the lane's row (a member's query head; zero past the
  // group), loaded while the first key tiles are in flight.
  u32x4 qb[kRowTiles][D / 32];
  int lim[kRowTiles];
  auto load_q = [&] {
#pragma unroll
    for (int nr = 0; nr < kRowTiles; ++nr) {
      const int row = wrow0 + 16 * nr + r16;
      const int mi = m0 + row / G;
      const int g = row - (row / G) * G;
      const bool valid = mi < members;
      lim[nr] = kend_wg - 1;
      const char* qrow = (const char*)p.q +
                         (((int64_t)(first + mi) * p.num_heads + (int64_t)head * G + g) * D) * 2 +
                         q4 * 16;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
        qb[nr][i] = valid ? *(const u32x4*)(qrow + 64 * i) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  attend_keys<D>(a, c, qb, lim, kstart, kend_wg, kend, kend, kfull, wave_rows, p.scale_log2, bad, buf,
                 wave, lane, load_q);
  if (!wave_rows) return;

#pragma unroll
  for (int nr = 0; nr < kRowTiles; ++nr) {
    const int row = wrow0 + 16 * nr + r16;
    const int mi = m0 + row / G;
    const int g = row - (row / G) * G;
    if (mi >= members) continue;
    const int64_t wslot =
        ((int64_t)(first + mi) * p.num_heads + (int64_t)head * G + g) * p.num_partitions + kp;
    // o[jt][rr] is head dim 16 jt + 4 q4 + rr of the lane's row
    float* orow = p.ws_o + wslot * D + 4 * q4;
#pragma unroll
    for (int jt = 0; jt < kVd; ++jt) *(f32x4*)(orow + 16 * jt) = a[nr].o[jt];
    if (q4 == 0) {
      p.ws_ml[wslot * 2 + 0] = a[nr].m;
      p.ws_ml[wslot * 2 + 1] = bad ? __builtin_nanf("") : a[nr].l[0];  // a bad table: NaN rows
    }
  }
}


// A work-group is one kind or the other, so the two share one LDS
// allocation: the prefix part's four staging buffers (64 KB at head_dim 128)
// or the decode work-group's merge space.  Two work-groups then fit a
// compute unit.
template <int D>
union SharedPrefixLds {
  unsigned char kv[kLdsBufs][kStepBytes<D>];
  DecodeLds<D> tail;
};

// Two resident work-groups per compute unit (both kinds fit 256 registers
// per lane; without the bound the allocator spends AGPRs and halves that).
// Work-group x: the prefix attention's work-group x while x < prefix_wgs (a
// multiple of 8, so x % 8 still names the XCD), then the tails.
template <int D>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void shared_prefix_kernel(DecodeParams p, int prefix_wgs) {
  __shared__ __attribute__((aligned(1024))) SharedPrefixLds<D> lds;
  const int x = blockIdx.x;
  if (x < prefix_wgs)
    prefix_wg<D>(p, x, lds.kv);
  else
    decode_wg<D, kModeTail>(p, x - prefix_wgs, lds.tail);
}

// Merge of each row's prefix partials (slots [0, kp), one per prefix
// partition) and tail partials (slots prefix.parts + [0, tp)):
//     out = sum_q w_q o_q / sum_q w_q l_q,  w_q = exp2(m_q - max_q m_q).
// One 256-thread work-group per (sequence, KV head); a thread owns four
// consecutive output elements of one query head and reads that head's
// partials itself.  Up to kMergeRegs partials are loaded into registers in
// one round together with the table check, so the work-group waits on two
// memory latencies (its length, then everything else); longer lists loop.  A
// member whose table does not start with its leader's prefix blocks, or whose
// length stops inside the prefix, gets a NaN row (the prefix partials are not
// its keys).
constexpr int kMergeThreads = 256;
constexpr int kMergeRegs = 8;

__device__ inline int merge_slot(const DecodeParams& p, int kp, int q) {
  return q < kp ? q : p.prefix.parts + (q - kp);
}

template <int D>
__global__ __launch_bounds__(kMergeThreads) void prefix_merge_kernel(DecodeParams p) {
  const int head = blockIdx.x % p.kv_heads;
  const int seq = blockIdx.x / p.kv_heads;
  const int len = p.seq_lens[seq];
  if (!seq_len_ok(p, len)) return;  // the tail work-group already wrote NaN
  const int grp = shared_prefix_group(p.prefix, seq);
  const int pfx = grp >= 0 ? p.prefix.tokens[grp] : 0;
  const int kp = pfx > 0 ? ceil_div_i(pfx, p.prefix.partition) : 0;
  const int tp = len > pfx ? ceil_div_i(len - pfx, p.partition_size) : 0;
  if (pfx == 0 && tp <= 1) return;  // the tail work-group wrote the row itself
  const int tid = threadIdx.x;
  const int G = p.group;
  const int n = kp + tp;
  const int64_t row0 = (int64_t)seq * p.num_heads + (int64_t)head * G;
  uint16_t* out = (uint16_t*)p.out;
  // the first item of this thread, loaded before the table check
  const int i0 = 4 * tid;
  const bool has0 = i0 < G * D;
  const int g0 = i0 / D;
  float m0[kMergeRegs], l0[kMergeRegs];
  f32x4 o0[kMergeRegs];
  if (has0 && n <= kMergeRegs) {
    const float* ml = p.ws_ml + (row0 + g0) * p.num_partitions * 2;
    const float* o = p.ws_o + (row0 + g0) * p.num_partitions * D + (i0 - g0 * D);
#pragma unroll
    for (int q = 0; q < kMergeRegs; ++q) {
      if (q < n) {
        const int slot = merge_slot(p, kp, q);
        m0[q] = ml[2 * slot];
        l0[q] = ml[2 * slot + 1];
        o0[q] = *(const f32x4*)(o + (int64_t)slot * D);
      }
    }
  }
  bool diff = pfx > 0 && len < pfx;
  if (pfx > 0) {
    const int32_t* mine = p.block_tables + (int64_t)seq * p.max_blocks_per_seq;
    const int32_t* lead = p.block_tables + (int64_t)p.prefix.start[grp] * p.max_blocks_per_seq;
    for (int j = tid; j < (pfx >> p.block_shift); j += kMergeThreads) diff |= mine[j] != lead[j];
  }
  const bool bad = __syncthreads_or(diff);
  for (int i = i0; i < G * D; i += 4 * kMergeThreads) {
    const int g = i / D;
    const int d = i - g * D;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
    if (i == i0 && n <= kMergeRegs) {
      float mx = -INFINITY;
#pragma unroll
      for (int q = 0; q < kMergeRegs; ++q)
        if (q < n) mx = fmaxf(mx, m0[q]);
#pragma unroll
      for (int q = 0; q < kMergeRegs; ++q) {
        if (q < n) {
          const float w = exp2f(m0[q] - mx);
          l += w * l0[q];
          acc += w * o0[q];
        }
      }
    } else {
      const float* ml = p.ws_ml + (row0 + g) * p.num_partitions * 2;
      const float* o = p.ws_o + (row0 + g) * p.num_partitions * D + d;
      float mx = -INFINITY;
      for (int q = 0; q < n; ++q) mx = fmaxf(mx, ml[2 * merge_slot(p, kp, q)]);
#pragma unroll 4
      for (int q = 0; q < n; ++q) {
        const int slot = merge_slot(p, kp, q);
        const float w = exp2f(ml[2 * slot] - mx);
        l += w * ml[2 * slot + 1];
        acc += w * *(const f32x4*)(o + (int64_t)slot * D);
      }
    }
    const float inv = bad ? __builtin_nanf("") : 1.0f / l;
    *(u32x2*)(out + (row0 + g) * D + d) =
        u32x2{pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)};
  }
}

}  // namespace

hipError_t launch_shared_prefix(const DecodeParams& p, int head_dim, hipStream_t stream) {
  const int64_t prefix_wgs = p.prefix.wg_start[p.prefix.num_groups];  // a multiple of 8
  const int64_t tail_wgs = (int64_t)(p.num_partitions - p.prefix.parts) * p.num_seqs * p.kv_heads;
  if (prefix_wgs + tail_wgs > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(prefix_wgs + tail_wgs));
  const dim3 block(kPfWaves * 64);
  if (head_dim == 128)
    shared_prefix_kernel<128><<<grid, block, 0, stream>>>(p, (int)prefix_wgs);
  else if (head_dim == 64)
    shared_prefix_kernel<64><<<grid, block, 0, stream>>>(p, (int)prefix_wgs);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_prefix_merge(const DecodeParams& p, int head_dim, hipStream_t stream) {
  if (p.group > 16 || head_dim % 4 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((int64_t)p.num_seqs * p.kv_heads));
  if (head_dim == 64)
    prefix_merge_kernel<64><<<grid, kMergeThreads, 0, stream>>>(p);
  else if (head_dim == 128)
    prefix_merge_kernel<128><<<grid, kMergeThreads, 0, stream>>>(p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
