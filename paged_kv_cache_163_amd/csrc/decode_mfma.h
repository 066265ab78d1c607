// Split-partition paged decode on the gfx950 matrix cores (bf16 storage,
// fp32 accumulation): the work of one work-group, shared by the decode
// kernel (decode_mfma.hip) and the shared-prefix launch (shared_prefix.hip).
//
// One work-group of NW waves per (sequence, KV head, partition), longest
// sequences first.  The partition is cut into 32-token steps (mfma_step.h);
// wave w takes steps w, w + NW, ...  Loads run one step ahead of the math
// (two register sets).  NW = 4 by default; the plan takes 2 when a split
// into equal partitions yields half as many work items as the GPU has wave
// slots, so each wave walks more steps per prologue and merge.  With WP
// ("wave per partition", for splits with at least as many items as wave
// slots) the NW waves of a work-group take NW consecutive partitions of one
// (sequence, KV head), each wave all the steps of its own partition, and each
// writes its own partial: no cross-wave merge.
// At the end the waves merge (m, l, O) through LDS; a single-partition
// sequence writes its normalised bf16 output directly, otherwise the partial
// goes to the workspace and decode_reduce.hip merges the partitions.
#pragma once

#include "mfma_step.h"

namespace pa {
namespace {

using namespace mfma;

// Default waves per work-group, and the minimum waves per SIMD the register
// allocation must leave room for (tuning knobs; 0 = compiler's choice).
#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif
#ifndef PA_MFMA_MIN_WAVES_PER_EU
#define PA_MFMA_MIN_WAVES_PER_EU 0
#endif
constexpr int kWaves = PA_MFMA_WAVES;

// Longest-first work order.  Hardware dispatches work-groups in index order,
// so giving the low indices to long sequences leaves short ones for the end
// of the launch and trims its tail (a host-sorted batch ran ~5 % faster).
// Every work-group derives the same order, a counting sort of the sequences
// into 256 length bins (longest bin first, index order inside a bin), and
// takes the sequence at its rank slot.  Wave 0 does the work (its LDS
// operations are ordered, so no barrier is needed until the hand-off);
// batches above kRankMaxSeqs keep index order.
constexpr int kRankMaxSeqs = 4096;
constexpr int kRankRegs = 8;  // lengths kept in registers per lane (batches <= 512)

// 256 length bins over [0, max_seq_len]; zero and unservable lengths go last.
__device__ inline int length_bin(int len, int max_len, float bins_per_token) {
  if (len <= 0 || len > max_len) return 0;
  return min(255, (int)((float)len * bins_per_token));
}

struct Ranked {
  int seq;
  int len;
};

__device__ inline Ranked ranked_seq(const DecodeParams& p, int slot, int* sm_hist,
                                   int* sm_pick) {
  const int tid = threadIdx.x;
  const int B = p.num_seqs;
  if (B > kRankMaxSeqs) return Ranked{slot, p.seq_lens[slot]};
  if (tid < 64) {
    const int lane = tid;
    const int maxl = p.max_seq_len;
    const float per_tok = 256.0f / ((float)maxl + 1.0f);
    int lens[kRankRegs];
#pragma unroll
    for (int j = 0; j < kRankRegs; ++j) {
      const int s = lane + 64 * j;
      lens[j] = s < B ? p.seq_lens[s] : -1;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) sm_hist[4 * lane + j] = 0;
#pragma unroll
    for (int j = 0; j < kRankRegs; ++j)
      if (lane + 64 * j < B) atomicAdd(&sm_hist[length_bin(lens[j], maxl, per_tok)], 1);
    for (int s = lane + 64 * kRankRegs; s < B; s += 64)
      atomicAdd(&sm_hist[length_bin(p.seq_lens[s], maxl, per_tok)], 1);
    // descending exclusive scan, 4 bins per lane (lane 0 holds the longest)
    int c[4], tot = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = sm_hist[255 - (4 * lane + j)];
      tot += c[j];
    }
    int incl = tot;
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int start = incl - tot, bin = -1, want = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (slot >= start && slot < start + c[j]) {
        bin = 255 - (4 * lane + j);
        want = slot - start;
      }
      start += c[j];
    }
    const uint64_t owner = __ballot(bin >= 0);
    const int src = __ffsll((unsigned long long)owner) - 1;
    bin = __shfl(bin, src);
    want = __shfl(want, src);
    // the want-th sequence of that bin, in index order (64 sequences per round)
    int seen = 0, pick = -1, pick_len = 0;
    for (int j = 0; 64 * j < B; ++j) {
      int len = -1;
#pragma unroll
      for (int r = 0; r < kRankRegs; ++r)
        if (r == j) len = lens[r];
      if (j >= kRankRegs && lane + 64 * j < B) len = p.seq_lens[lane + 64 * j];
      const bool match = lane + 64 * j < B && length_bin(len, maxl, per_tok) == bin;
      const uint64_t m = __ballot(match);
      const int n = __popcll(m);
      if (want < seen + n) {
        const int before = seen + __popcll(m & ((1ull << lane) - 1));
        if (match && before == want) {
          pick = lane + 64 * j;
          pick_len = len;
        }
        break;
      }
      seen += n;
    }
    const uint64_t found = __ballot(pick >= 0);
    const int from = __ffsll((unsigned long long)found) - 1;
    pick = __shfl(pick, from);
    pick_len = __shfl(pick_len, from);
    if (lane == 0) {
      sm_pick[0] = pick;
      sm_pick[1] = pick_len;
    }
  }
  __syncthreads();
  // wave-uniform: keep the sequence and its length in scalar registers
  return Ranked{__builtin_amdgcn_readfirstlane(sm_pick[0]),
                __builtin_amdgcn_readfirstlane(sm_pick[1])};
}

// kModePlain: one per-layer pool.  kModeFused: plus the step's append.
// kModeLayered: one or more layers of a layered pool (layer = blockIdx.y).
// kModeOrdered: a per-layer pool with the caller's longest-first order.
// kModeFusedOrdered: kModeFused in the caller's order.
// kModeTail: shared-prefix decode; each sequence's partitions start after
// its group's shared prefix (the prefix work-groups of shared_prefix.hip
// cover the prefix), in the caller's order when one is given (else index
// order), and every partial goes to the workspace unless the sequence has no
// prefix and one partition.
enum Mode { kModePlain, kModeFused, kModeLayered, kModeOrdered, kModeTail, kModeFusedOrdered };

// The LDS of one decode work-group, declared by the kernel that runs it (the
// shared-prefix launch overlays it with the prefix work-groups' staging).
template <int D, int NW = kWaves>
struct DecodeLds {
  float o[NW][16][D];      // per-wave (m, l, O) for the cross-wave merge
  float m[NW][16];
  float l[NW][16];
  int hist[256];           // longest-first ranking
  int pick[2];
  __attribute__((aligned(16))) unsigned char nw[2 * D * 2];  // fused append: the new K and V rows
};

// The work of decode work-group `wg` (sequence, KV head, partition; with WP
// partitions NW*part .. NW*part + NW - 1) in mode M, with NW waves.
template <int D, int M, int NW = kWaves, bool WP = false>
__device__ __forceinline__ void decode_wg(const DecodeParams& p, int wg, DecodeLds<D, NW>& lds) {
  constexpr int kKi = D / 32;
  constexpr bool kFused = M == kModeFused || M == kModeFusedOrdered;
  static_assert(!(WP && (kFused || M == kModeTail)), "wave-per-partition: plain modes only");
  auto& sm_o = lds.o;
  auto& sm_m = lds.m;
  auto& sm_l = lds.l;
  int* sm_hist = lds.hist;
  int* sm_pick = lds.pick;
  unsigned char* sm_new = lds.nw;
  WorkItem w = decode_work_item(p, wg);
  Ranked rk;
  if constexpr (M == kModeOrdered || M == kModeFusedOrdered) {
    // the caller's order; an entry outside the batch leaves its slot idle
    rk.seq = p.order[w.seq];
    if (rk.seq < 0 || rk.seq >= p.num_seqs) return;
    rk.len = p.seq_lens[rk.seq];
  } else if constexpr (M == kModeTail) {
    // the caller's order (longest tail first) or index order; an entry
    // outside the batch leaves its slot idle
    rk.seq = p.order != nullptr ? p.order[w.seq] : w.seq;
    if (rk.seq < 0 || rk.seq >= p.num_seqs) return;
    rk.len = p.seq_lens[rk.seq];
  } else {
    rk = ranked_seq(p, w.seq, sm_hist, sm_pick);
  }
  w.seq = rk.seq;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15;
  const int q4 = lane >> 4;
  const int G = p.group;
  const int len = rk.len;
  const int64_t out_row0 = (int64_t)w.seq * p.num_heads + (int64_t)w.head * G;
  const char* qbase = (const char*)p.q;
  const char* kcache = (const char*)p.k_cache;
  const char* vcache = (const char*)p.v_cache;
  uint16_t* out = (uint16_t*)p.out;
  float* ws_o = p.ws_o;
  float* ws_ml = p.ws_ml;
  if constexpr (M == kModeLayered) {
    const int64_t layer = blockIdx.y;
    qbase += layer * p.layer_q_stride * 2;
    out += layer * p.layer_q_stride;
    kcache += layer * p.layer_kv_stride * 2;
    vcache += layer * p.layer_kv_stride * 2;
    if (ws_o != nullptr) {
      ws_o += layer * p.layer_ws_stride;
      ws_ml += layer * (p.layer_ws_stride / D) * 2;
    }
  }

  if (!seq_len_ok(p, len) || len == 0) {
    if (w.part == 0) {
      const uint16_t fill = len == 0 ? (uint16_t)0 : (uint16_t)0x7FC0;
      for (int i = tid; i < G * D; i += NW * 64) out[out_row0 * D + i] = fill;
      if (kFused) store_new_token(p, w.seq, w.head, D * 2, tid);
    }
    return;
  }
  // Shared-prefix decode: positions before `pfx` belong to the prefix kernel.
  int pfx = 0;
  if constexpr (M == kModeTail) pfx = shared_prefix_tokens(p.prefix, w.seq);
  // this wave's (WP) or this work-group's partition
  const int part = WP ? w.part * NW + wave : w.part;
  // part * partition_size < max_seq_len by the plan; the sum with the prefix
  // is formed in 64 bits.  A WP wave past the last partition has no work (no
  // barrier follows in that mode).
  const int64_t pstart64 = (int64_t)pfx + (int64_t)part * p.partition_size;
  if (pstart64 >= len) return;
  const int pstart = (int)pstart64;
  const int pend = range_end(pstart, p.partition_size, len);
  const int nparts = ceil_div_i(len - pfx, p.partition_size);
  // Fused append: the new token is position len - 1, in the last partition.
  // Its work-group takes the token's K and V from the new rows instead of the
  // cache slot (patched into the loaded step, before its math, by the wave
  // whose step holds the token), so the decode is exactly the plain decode of
  // the appended cache; that wave writes the rows to the slot after its last
  // cache read.  It fetches the rows (lanes 0 .. kNewParts-1) up front and
  // keeps them in LDS (sm_new, its own) rather than in registers.
  constexpr int kNewParts = D / 4;  // 16-byte parts of the K and V rows
  int new_pos = -1;                 // the new token's position, if in this partition
  int new_wave = -1;                // the wave whose step holds it
  int64_t new_slot = -1;
  nt_u32x4 new_part = {0u, 0u, 0u, 0u};
  if constexpr (kFused) {
    const NewToken nt = new_token(p, w.seq, w.head, len, D * 2);
    if (nt.pos >= pstart && nt.pos < pend) {
      new_pos = nt.pos;
      new_slot = nt.slot;
      new_wave = ((nt.pos - pstart) >> 5) % NW;
      if (wave == new_wave && lane < kNewParts)
        new_part = new_row_part(p, w.seq, w.head, D * 2, lane);
    }
  }

  // Q^T as the B operand: column r16 = query head h*G + r16, zero when r16 >= G.
  u32x4 qb[kKi];
  {
    const char* qrow = qbase + ((out_row0 + r16) * D) * 2 + q4 * 16;
#pragma unroll
    for (int i = 0; i < kKi; ++i)
      qb[i] = r16 < G ? *(const u32x4*)(qrow + 64 * i) : u32x4{0u, 0u, 0u, 0u};
  }

  SeqView c;
  const int64_t head_stride = (int64_t)p.block_size * D * 2;
  c.kbase = kcache + (int64_t)w.head * head_stride;
  c.vbase = vcache + (int64_t)w.head * head_stride;
  c.table = p.block_tables + (int64_t)w.seq * p.max_blocks_per_seq;
  c.block_stride = M == kModeLayered ? p.block_stride * 2 : (int64_t)p.kv_heads * head_stride;
  c.nblocks_valid = (len + p.block_size - 1) >> p.block_shift;
  c.num_blocks = p.num_blocks;
  c.block_shift = p.block_shift;
  c.bmask = p.block_size - 1;

  Acc<D> a;
  reset(a);
  bool bad = false;

  // Two register sets, loads one step ahead of the math; tokens >= pend masked.
  const int stride = WP ? 32 : 32 * NW;
  int base = WP ? pstart : pstart + 32 * wave;
  if (base < pend) {
    StepRegs<D> ra, rb;
    load_step<D>(ra, c, base, r16, q4, bad);
    if (kFused && wave == new_wave && lane < kNewParts)
      *(nt_u32x4*)(sm_new + 16 * lane) = new_part;
    while (true) {
      int next = base + stride;
      if (next < pend) load_step<D>(rb, c, next, r16, q4, bad);
      if (kFused && wave == new_wave && new_pos >= base && new_pos < base + 32)
        patch_new_token<D>(ra, sm_new, new_pos - base, r16, q4);
      compute_step<D>(ra, a, qb, base, pend, p.scale_log2, q4);
      base = next;
      if (base >= pend) break;
      next = base + stride;
      if (next < pend) load_step<D>(ra, c, next, r16, q4, bad);
      if (kFused && wave == new_wave && new_pos >= base && new_pos < base + 32)
        patch_new_token<D>(rb, sm_new, new_pos - base, r16, q4);
      compute_step<D>(rb, a, qb, base, pend, p.scale_log2, q4);
      base = next;
      if (base >= pend) break;
    }
  }
  finish_wave(a, bad);
  stash_wave<D, NW>(a, sm_o, sm_m, sm_l, wave, r16, q4, G);
  if constexpr (WP) {
    // each wave stores its own partition's result from its own stash (one
    // wave's LDS operations complete in order)
    // in 16-byte parts: four consecutive head dims per lane and store
    __builtin_amdgcn_wave_barrier();
    for (int i = 4 * lane; i < G * D; i += 4 * 64) {
      const int g = i / D;
      const int d = i - g * D;
      const f32x4 o = *(const f32x4*)&sm_o[wave][g][stash_col<D>(g, d)];
      const float l = sm_l[wave][g];
      if (nparts == 1) {
        const float inv = 1.0f / l;
        *(u32x2*)(out + (out_row0 + g) * D + d) =
            u32x2{(uint32_t)f32_to_bf16(o[0] * inv) | ((uint32_t)f32_to_bf16(o[1] * inv) << 16),
                  (uint32_t)f32_to_bf16(o[2] * inv) | ((uint32_t)f32_to_bf16(o[3] * inv) << 16)};
      } else {
        const int64_t slot = (out_row0 + g) * p.num_partitions + part;
        *(f32x4*)(ws_o + slot * D + d) = o;
        if (d == 0) {
          ws_ml[slot * 2 + 0] = sm_m[wave][g];
          ws_ml[slot * 2 + 1] = l;
        }
      }
    }
    return;
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += NW * 64) {
    const int g = i / D;
    const int d = i - g * D;
    float mx, l, o;
    merge_waves<D, NW>(sm_o, sm_m, sm_l, g, d, mx, l, o);
    if (nparts == 1 && pfx == 0) {
      out[(out_row0 + g) * D + d] = f32_to_bf16(o / l);
    } else {
      const int part_slot = M == kModeTail ? p.prefix.parts + w.part : w.part;
      const int64_t slot = (out_row0 + g) * p.num_partitions + part_slot;
      ws_o[slot * D + d] = o;
      if (d == 0) {
        ws_ml[slot * 2 + 0] = mx;
        ws_ml[slot * 2 + 1] = l;
      }
    }
  }
  if (kFused && wave == new_wave && lane < kNewParts)
    store_row_part(p, new_slot, w.head, D * 2, lane, *(const nt_u32x4*)(sm_new + 16 * lane));
}

}  // namespace
}  // namespace pa
