// The 128-row tile engine of the matrix-core attention kernels that share
// K/V tiles across many query rows: chunked prefill (prefill_mfma.hip) and the
// prefix part of the shared-prefix decode (shared_prefix.hip).
//
// A work-group of kPfWaves waves covers kPrefillRows query rows of one KV
// head; each wave owns kRowTiles 16-row column tiles of the MFMA step from
// mfma_step.h (S^T = K Q^T, O^T += V^T P^T) with its Q^T operands in
// registers.  The work-group walks the keys in 32-token steps (attend_keys)
// and stages each step's K and V tiles in LDS once for all its waves, so each
// K/V byte is fetched once per work-group: gfx950's global-to-LDS loads fill
// four LDS buffers three steps ahead of the math, with no register on the
// way.  Row limits are per lane (a lane's score column is one row); V rows
// past a wave's last key are zeroed so tail slots never reach the sum.  The
// steps a wave's rows all see whole come first and take an unmasked step;
// the remaining steps take the masked one.
#pragma once

#include "mfma_step.h"

namespace pa {
namespace {

using namespace mfma;

constexpr int kPfWaves = 4;
constexpr int kRowTiles = 2;                 // 16-row MFMA column tiles per wave
constexpr int kWaveRows = 16 * kRowTiles;
static_assert(kPfWaves * kWaveRows == kPrefillRows, "work-group rows");

// A row's running state: O^T tiles, the row sum (computed on the matrix core
// as P^T against a ones operand, so it is the exact sum of the bf16 P the
// output uses; all four elements hold the lane's row sum) and the reference
// max the probabilities are taken against (base-2 units).
template <int D>
struct PfAcc {
  f32x4 o[D / 16];
  f32x4 l;
  float m;
  float thr;  // m + kSlack: a step max above it rescales
};

// How far (base-2 units) a row's step max may rise above its reference max
// before O and l are rescaled: probabilities stay <= 2^8, harmless in fp32 and
// bf16, and most steps skip the rescale of the accumulators.
constexpr float kSlack = 8.0f;

// Compile-time choice of the masked or unmasked step.
template <bool B>
struct MaskTag {
  static constexpr bool value = B;
};

// Max over the four lanes that share r16 (one per 16-lane row of the wave).
// The maxes here and in the step are the NaN-propagating maximum
// (v_maximum3_f32): unlike fmaxf's maxnum it needs no quieting of its
// operands, and on the scores (never NaN) the two agree.
__device__ inline float row_max4(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ inline uint32_t pack_bf16(float lo, float hi) {  // round to nearest even
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Softmax and PV of one 32-key step for all row tiles of a wave, from its
// raw scores s.  kMask (a step that some row of the wave does not see whole:
// it reaches past kfull, the wave's first row position) masks keys > lim[nr]
// (the lane's row position); if the step also reaches kvalid, the first key
// that may hold anything but finite data (tail slots past the sequence), it
// zeroes the V values of keys from there on, since a zero probability times
// a NaN would still reach the sum.  Unmasked steps need neither.  The row
// tiles go through the step together with one wave-uniform rescale branch,
// so their dependent max and exp chains interleave.
// c = scale * log2(e) > 0 (the host rejects other scales), so c times a max
// of s is the max of c*s, rounding included (rounding is monotonic).  The
// rescale test therefore needs only each lane's own max: a row's max over
// its four lanes exceeds the threshold exactly when one lane's does, and the
// lane exchange runs only inside the (rare) rescale branch.  A row tile
// whose keys are all masked in a step has a max of -inf: its reference max
// stays and its probabilities are 0 (every tile sees a finite key in its
// first step).
template <int D, bool kMask>
__device__ inline void step_softmax_pv(const f32x4 (&s)[kRowTiles][2], u32x4 (&av)[D / 16],
                                       PfAcc<D> (&a)[kRowTiles], int base, int kvalid,
                                       const int (&lim)[kRowTiles], float c, int q4,
                                       const u32x4& ones) {
  constexpr int kVd = D / 16;
  float sv[kRowTiles][8];
#pragma unroll
  for (int nr = 0; nr < kRowTiles; ++nr)
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[nr][e] = s[nr][e >> 2][e & 3];
  if constexpr (kMask) {
    if (base + 32 > kvalid) {  // wave-uniform: the step reaches past the live keys
      uint32_t keep[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int tok = base + 16 * (u >> 1) + 4 * q4 + 2 * (u & 1);
        keep[u] = (tok < kvalid ? 0x0000FFFFu : 0u) | (tok + 1 < kvalid ? 0xFFFF0000u : 0u);
      }
#pragma unroll
      for (int jt = 0; jt < kVd; ++jt)
#pragma unroll
        for (int u = 0; u < 4; ++u) av[jt][u] &= keep[u];
    }
#pragma unroll
    for (int nr = 0; nr < kRowTiles; ++nr)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = base + 16 * (e >> 2) + 4 * q4 + (e & 3);
        sv[nr][e] = tok <= lim[nr] ? sv[nr][e] : -INFINITY;
      }
  }
  float mr[kRowTiles];
  bool grow = false;
#pragma unroll
  for (int nr = 0; nr < kRowTiles; ++nr) {
    mr[nr] = sv[nr][0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mr[nr] = __builtin_elementwise_maximum(mr[nr], sv[nr][e]);
    grow |= mr[nr] * c > a[nr].thr;
  }
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // wave-uniform
#pragma unroll
    for (int nr = 0; nr < kRowTiles; ++nr) {
      const float m_new = fmaxf(a[nr].m, row_max4(mr[nr]) * c);
      const float keep = __builtin_amdgcn_exp2f(a[nr].m - m_new);  // 0 on the first step
#pragma unroll
      for (int jt = 0; jt < kVd; ++jt) a[nr].o[jt] *= keep;
      a[nr].l *= keep;
      a[nr].m = m_new;
      a[nr].thr = m_new + kSlack;
    }
  }
  // Tile 0's probabilities first.  Its products then go to the matrix cores a
  // few at a time, each group followed by one packed pair of tile 1's
  // exponentials: the products do not depend on them, so the wave keeps the
  // matrix and vector pipes busy at once instead of one after the other.
  static_assert(kRowTiles == 2 && kVd % 4 == 0, "two row tiles, whole groups");
  u32x4 pb[kRowTiles];
  auto probs = [&](int nr, int u) {
    pb[nr][u] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(sv[nr][2 * u], c, -a[nr].m)),
                          __builtin_amdgcn_exp2f(fmaf(sv[nr][2 * u + 1], c, -a[nr].m)));
  };
#pragma unroll
  for (int u = 0; u < 4; ++u) probs(0, u);
  a[0].l = mma(ones, pb[0], a[0].l);
#pragma unroll
  for (int jt = 0; jt < kVd; ++jt) {
    __builtin_amdgcn_sched_barrier(0);
    a[0].o[jt] = mma(av[jt], pb[0], a[0].o[jt]);
    if (jt % (kVd / 4) == kVd / 4 - 1) {
      probs(1, jt / (kVd / 4));
      asm volatile("" : "+v"(pb[1][jt / (kVd / 4)]));  // computed here, not at its use
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  a[1].l = mma(ones, pb[1], a[1].l);
#pragma unroll
  for (int jt = 0; jt < kVd; ++jt) a[1].o[jt] = mma(av[jt], pb[1], a[1].o[jt]);
}

// Direct global-to-LDS staging (global_load_lds_dwordx4).  One instruction
// moves 16 bytes per lane straight into LDS: lane l's bytes land at the
// wave-uniform LDS address + 16 l, so each instruction fills one contiguous
// 1 KiB block.  A step's K and V tiles are D/16 such blocks each (K first).
// Every block comes from one 16-token tile of the cache (rows 16 h .. 16 h +
// 15 of the step), so an instruction reads from one wave-uniform base
// address in scalar registers plus a fixed 32-bit offset per lane, and the
// step's address arithmetic stays on the scalar unit.  Block h * D/32 + j of
// a tile holds the 16-byte chunks 4j .. 4j + 3 of those 16 rows, chunk
// 4j + cc of row r at lane
//   16 cc + r                   in a K block,
//   16 cc + (r ^ 8 (cc & 1))    in a V block.
// Measured with a bank-conflict probe on gfx950: the K operand reads
// (ds_read_b128, 16 rows of one chunk) are then one contiguous 1 KiB and
// conflict-free; the V transpose reads (ds_read_b64_tr_b16, rows 0..7 of two
// adjacent chunks per half-wave) are conflict-free with the XOR and 2-way
// without it.  Wave w issues blocks w, w + kPfWaves, ... of a step.
constexpr int kLdsBufs = 4;                        // LDS buffers; steps staged ahead: 3
template <int D>
constexpr int kTileBytes = 32 * D * 2;             // one K or V tile of a step
template <int D>
constexpr int kStepBytes = 2 * kTileBytes<D>;
template <int D>
constexpr int kDmaPerWave = kStepBytes<D> / 1024 / kPfWaves;
static_assert(kStepBytes<64> % (1024 * kPfWaves) == 0, "whole blocks per wave");

typedef __attribute__((address_space(3))) void lds_void;

// A lane's fixed part of its staging addresses.
template <int D>
struct DmaLane {
  uint32_t off[kDmaPerWave<D>];  // byte offset inside the 16-token block tile
  bool v[kDmaPerWave<D>];        // wave-uniform: the instruction stages V
  bool hi[kDmaPerWave<D>];       // wave-uniform: it stages the step's second 16-token tile
};

template <int D>
__device__ inline DmaLane<D> dma_lane(int wave, int lane) {
  constexpr int kPer = D / 32;  // 1 KiB blocks per 16-token tile of K or V
  DmaLane<D> dl;
  const int cc = lane >> 4;
  const int s16 = lane & 15;
#pragma unroll
  for (int u = 0; u < kDmaPerWave<D>; ++u) {
    const int bi = u * kPfWaves + wave;
    dl.v[u] = bi >= 2 * kPer;
    const int kb = dl.v[u] ? bi - 2 * kPer : bi;
    dl.hi[u] = kb >= kPer;
    const int j = kb % kPer;
    const int rr = dl.v[u] ? s16 ^ (8 * (cc & 1)) : s16;  // row in the 16-token tile
    dl.off[u] = (uint32_t)(rr * (D * 2) + 16 * (4 * j + cc));
  }
  return dl;
}

// Two block-table entries through the scalar cache.  The compiler would read
// them with vector loads (the staging instructions count as possible writes to
// global memory), whose waits would also wait for the staging in flight.
__device__ inline void table_pair(int (&phys)[2], const int32_t* a, const int32_t* b) {
  int x, y;
  asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(x), "=&s"(y)
               : "s"(a), "s"(b)
               : "memory");
  phys[0] = x;
  phys[1] = y;
}

// Work-group barrier that orders LDS only: the staging instructions in flight
// (counted by vmcnt) are waited for explicitly by dma_wait, not here.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One 16-byte-per-lane direct load into LDS (lane l's bytes at lds + 16 l;
// M0 holds the wave-uniform LDS address and is restored afterwards) from the
// wave-uniform address `base` plus the lane's 32-bit offset.
// Written as inline assembly so that the compiler does not track it: its own
// tracking waits for every staging load in flight before the LDS transpose
// reads of any buffer.  Completion is awaited explicitly (dma_wait) before a
// buffer is read.
__device__ inline void dma16(const char* base, uint32_t off, unsigned char* lds) {
  const uint32_t m = (uint32_t)(uintptr_t)(lds_void*)lds;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(m)
      : "memory");
}

// Issue the wave's kDmaPerWave blocks of the step at key `base` into the LDS
// buffer `buf`.  Keys past the sequence re-read its last live block (masked
// later); a table entry outside the pool sets `bad` (work-group uniform) and
// reads block 0 instead.
template <int D>
__device__ inline void dma_issue(const DmaLane<D>& dl, const SeqView& c, int wave, int base,
                                 bool& bad, unsigned char* buf) {
  int phys[2];
  table_pair(phys, c.table + min(base >> c.block_shift, c.nblocks_valid - 1),
             c.table + min((base + 16) >> c.block_shift, c.nblocks_valid - 1));
  int64_t tile[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int tok0 = base + 16 * kt;
    if (phys[kt] < 0 || phys[kt] >= c.num_blocks) {
      bad = true;
      phys[kt] = 0;
    }
    tile[kt] = (int64_t)phys[kt] * c.block_stride + (int64_t)(tok0 & c.bmask) * (D * 2);
  }
#pragma unroll
  for (int u = 0; u < kDmaPerWave<D>; ++u) {
    const int bi = u * kPfWaves + wave;
    // When each 16-token tile of K or V is kPfWaves blocks (head_dim 128),
    // instruction u of every wave stages the same kind of block: K for the
    // first half of the instructions, V for the second, the step's second
    // tile for odd u.  The choice is then a compile-time one, with no scalar
    // selects per instruction.
    constexpr bool kFixed = D / 32 == kPfWaves;
    const bool v = kFixed ? u >= kDmaPerWave<D> / 2 : dl.v[u];
    const bool hi = kFixed ? (u & 1) != 0 : dl.hi[u];
    dma16((v ? c.vbase : c.kbase) + (hi ? tile[1] : tile[0]), dl.off[u], buf + 1024 * bi);
  }
}

// Byte offsets of lane (r16, q4)'s K operand reads (row 16 kt + r16, chunk
// 4 i + q4, at + 1024 (kt D/32 + i)) and V transpose reads (key 4 q4 + r16 / 4
// (+ 16), head dims 16 jt + 4 (r16 % 4) .. + 3, at + 1024 (jt / 2) + 512 (jt
// % 2) (+ 1024 D/32)) in a staged step; the V offset is relative to the V
// tile.
__device__ inline uint32_t dma_k_lane(int r16, int q4) {
  return 16 * (16 * q4 + r16);
}
__device__ inline uint32_t dma_v_lane(int r16, int q4) {
  const int b = (r16 >> 1) & 1;
  const int R = 4 * q4 + (r16 >> 2);
  return 16 * (16 * b + (R ^ (8 * b))) + 8 * (r16 & 1);
}

// Scores S^T = K Q^T of one 32-key step for every row tile of a wave, raw
// (unscaled): s[nr][kt][j] is key 16 kt + 4 q4 + j of the step for the
// lane's row of tile nr.  K: lane (r16, q4) reads row 16 kt + r16, head dims
// 32 i + 8 q4 .. + 7, once for all row tiles; `ks` is the step's buffer plus
// dma_k_lane.
template <int D>
__device__ inline void step_scores(f32x4 (&s)[kRowTiles][2], const unsigned char* ks,
                                  const u32x4 (&qb)[kRowTiles][D / 32]) {
#pragma unroll
  for (int nr = 0; nr < kRowTiles; ++nr)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[nr][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 k[D / 32][2];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) k[i][kt] = *(const u32x4*)(ks + 1024 * (kt * (D / 32) + i));
  // Tile 0 first: its running max can then be taken while tile 1's products run.
#pragma unroll
  for (int nr = 0; nr < kRowTiles; ++nr)
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) s[nr][kt] = mma(k[i][kt], qb[nr][i], s[nr][kt]);
}

// The V^T operands of one step (A operands of the PV MFMAs).  Tile jt covers
// head dims 16 jt .. 16 jt + 15: lane (r16, q4) holds d = 16 jt + r16 for the
// step's keys tau(q4, e) = 16 (e / 4) + 4 q4 + e % 4, e = 0..7, the order
// the score tiles leave P^T in.  The LDS transpose read (ds_read_b64_tr_b16)
// hands lane 4 b + c of each 16-lane group element c of the 8-byte rows that
// lanes b, b + 4, b + 8 and b + 12 of the group address; lane (r16, q4)
// addresses key 4 q4 + r16 / 4 (16 more for the second read) at head dims
// 16 jt + 4 (r16 % 4) .. + 3 (`v0`: the step's V tile plus dma_v_lane).
template <int D>
__device__ inline void read_v(u32x4 (&av)[D / 16], const unsigned char* v0) {
#pragma unroll
  for (int jt = 0; jt < D / 16; ++jt) {
    const unsigned char* p = v0 + 1024 * (jt >> 1) + 512 * (jt & 1);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 1024 * (D / 32)));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
    av[jt] = u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
}

// Wait for this wave's staging of the current step, leaving the `later`
// (0, 1 or 2) following steps' kDmaPerWave instructions each in flight.  The
// count is exact because vector loads complete in order and the key loop
// issues no other vector memory instruction after the first staging
// (another load would only make the wait stricter).
template <int D>
__device__ inline void dma_wait(int later) {
  if (later >= 2)
    __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * kDmaPerWave<D>) & 15) | (((2 * kDmaPerWave<D>) >> 4) << 14));
  else if (later == 1)
    __builtin_amdgcn_s_waitcnt(0x0F70 | (kDmaPerWave<D> & 15));
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);
}


// The work-group's walk over keys [kstart, kend_wg) in 32-key steps (kstart a
// multiple of 32).  Step t sits in buffer t % kLdsBufs.  Opening step t means:
// wait for this wave's part of its tiles, make every wave's part visible
// (barrier), and stage step t + 3 into the buffer every wave finished reading
// before that barrier.  The first two steps are requested before load_q()
// issues the Q loads, so the latencies overlap; the loads are all waited for
// before the walk, whose only vector memory instructions are then the staging.
// A wave takes the math of the steps below its own kend only; every wave
// stages and meets every barrier.  kfull is the wave's first row position:
// the steps at or before it need no mask.
template <int D, class LoadQ>
__device__ inline void attend_keys(PfAcc<D> (&a)[kRowTiles], const SeqView& c,
                                   const u32x4 (&qb)[kRowTiles][D / 32],
                                   const int (&lim)[kRowTiles], int kstart, int kend_wg,
                                   int kend, int kvalid, int kfull, bool wave_rows,
                                   float scale_log2,
                                   bool& bad, unsigned char (*buf)[kStepBytes<D>], int wave,
                                   int lane, LoadQ&& load_q) {
  const int r16 = lane & 15;
  const int q4 = lane >> 4;
  const DmaLane<D> dl = dma_lane<D>(wave, lane);
  const uint32_t kl = dma_k_lane(r16, q4);
  const uint32_t vl = kTileBytes<D> + dma_v_lane(r16, q4);
  // The row sums' ones operand, held in registers for the whole walk.
  u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  asm volatile("" : "+v"(ones));
  const int nsteps = (kend_wg - kstart + 31) >> 5;
  if (nsteps <= 0) {  // no keys: nothing staged, so nothing in flight at exit
    load_q();
    return;
  }
  dma_issue<D>(dl, c, wave, kstart, bad, buf[0]);
  if (nsteps > 1) dma_issue<D>(dl, c, wave, kstart + 32, bad, buf[1]);
  load_q();
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (nsteps > 2) dma_issue<D>(dl, c, wave, kstart + 64, bad, buf[2]);
  auto run = [&](int t, auto tag) {
    constexpr bool kMask = decltype(tag)::value;
    dma_wait<D>(min(nsteps - 1 - t, 2));
    lds_barrier();
    if (t + 3 < nsteps)
      dma_issue<D>(dl, c, wave, kstart + 32 * (t + 3), bad, buf[(t + 3) % kLdsBufs]);
    const int base = kstart + 32 * t;
    if (!kMask || base < kend) {
      const unsigned char* cur = buf[t % kLdsBufs];
      f32x4 s[kRowTiles][2];
      step_scores<D>(s, cur + kl, qb);
      u32x4 av[D / 16];
      read_v<D>(av, cur + vl);
      step_softmax_pv<D, kMask>(s, av, a, base, kvalid, lim, scale_log2, q4, ones);
    }
  };
  // Unmasked steps: base + 31 <= kfull (then also base < kend).  They come in
  // a loop of their own, which keeps the register assignments of the two step
  // kinds apart (one loop with both behind a branch spilled).
  const int nfull =
      wave_rows && kfull - kstart >= 31 ? min(nsteps, (kfull - kstart - 31) / 32 + 1) : 0;
  int t = 0;
  for (; t < nfull; ++t) run(t, MaskTag<false>{});
  for (; t < nsteps; ++t) run(t, MaskTag<true>{});
}

}  // namespace
}  // namespace pa
