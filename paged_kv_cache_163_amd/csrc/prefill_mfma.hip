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
// in 32-token steps: every thread loads 16-byte parts of the next step's K
// and V tiles from HBM while the waves compute the current one from LDS
// (double-buffered, one barrier per step), so each K/V byte is fetched once
// per work-group.  A wave whose rows end earlier skips the math of the later
// steps.  The causal limit is per lane (a lane's score column is one row); V
// rows past the wave's last key are zeroed so tail slots never reach the
// sum.  The first step holds key 0, which every row sees, so no row's
// running max stays -inf after it.
//
// Work order: work-group x runs on XCD x % 8.  All query tiles of one
// (sequence, KV head) pair are given consecutive slots on one XCD, latest
// tile (most keys) first, so the pair's K/V stays in that XCD's L2 while its
// tiles run.
#include "mfma_step.h"

namespace pa {
namespace {

using namespace mfma;

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kRowTiles = 2;                 // 16-row MFMA column tiles per wave
constexpr int kWaveRows = 16 * kRowTiles;
static_assert(kPfWaves * kWaveRows == kPrefillRows, "work-group rows");
// LDS bytes per staged K or V row: padding moves consecutive rows to other
// banks, so the lanes that read one 16-byte column of 16 rows collide less
// (32 bytes measured best of 0, 16, 32, 48 and 64).
template <int D>
constexpr int kKvStride = D * 2 + 32;
template <int D>
constexpr int kRowParts = D * 2 / 16;        // 16-byte parts of a K or V row
template <int D>
constexpr int kStageParts = 2 * 32 * kRowParts<D> / kPfThreads;  // per thread per step
static_assert(2 * 32 * kRowParts<128> % kPfThreads == 0 && 2 * 32 * kRowParts<64> % kPfThreads == 0,
              "every thread stages whole parts");

// A row's running state: O^T tiles, the row sum (computed on the matrix core
// as P^T against a ones operand, so it is the exact sum of the bf16 P the
// output uses; all four elements hold the lane's row sum) and the reference
// max the probabilities are taken against (base-2 units).
template <int D>
struct PfAcc {
  f32x4 o[D / 16];
  f32x4 l;
  float m;
};

// How far (base-2 units) a row's step max may rise above its reference max
// before O and l are rescaled: probabilities stay <= 2^8, harmless in fp32 and
// bf16, and most steps skip the rescale of the accumulators.
constexpr float kSlack = 8.0f;

// Max over the four lanes that share r16 (one per 16-lane row of the wave).
__device__ inline float row_max4(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ inline uint32_t pack_bf16(float lo, float hi) {  // round to nearest even
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Scores S^T = K Q^T of one 32-key step for every row tile of a wave, raw
// (unscaled): s[nr][kt][j] is key 16 kt + 4 q4 + j of the step for the
// lane's row of tile nr.  K: lane (r16, q4) reads staged row 16 kt + r16,
// head dims 32 i + 8 q4 .. + 7, once for all row tiles.
template <int D>
__device__ inline void step_scores(f32x4 (&s)[kRowTiles][2], const unsigned char* ks,
                                   const u32x4 (&qb)[kRowTiles][D / 32], int r16, int q4) {
#pragma unroll
  for (int nr = 0; nr < kRowTiles; ++nr)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[nr][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const u32x4 k = *(const u32x4*)(ks + (16 * kt + r16) * kKvStride<D> + 64 * i + 16 * q4);
#pragma unroll
      for (int nr = 0; nr < kRowTiles; ++nr) s[nr][kt] = mma(k, qb[nr][i], s[nr][kt]);
    }
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// The V^T operands of one step (A operands of the PV MFMAs).  Tile jt covers
// head dims 16 jt .. 16 jt + 15: lane (r16, q4) holds d = 16 jt + r16 for the
// step's keys tau(q4, e) = 16 (e / 4) + 4 q4 + e % 4, e = 0..7, the order
// the score tiles leave P^T in.  The LDS transpose read (ds_read_b64_tr_b16)
// hands lane 4 b + c of each 16-lane group element c of the 8-byte rows that
// lanes b, b + 4, b + 8 and b + 12 of the group address; lane (r16, q4)
// addresses key 4 q4 + r16 / 4 (16 more for the second read) at head dims
// 16 jt + 4 (r16 % 4) .. + 3.
template <int D>
__device__ inline void read_v(u32x4 (&av)[D / 16], const unsigned char* vs, int r16, int q4) {
  const unsigned char* v0 = vs + (4 * q4 + (r16 >> 2)) * kKvStride<D> + 8 * (r16 & 3);
#pragma unroll
  for (int jt = 0; jt < D / 16; ++jt) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + 32 * jt));
    const i16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + 16 * kKvStride<D> + 32 * jt));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
    av[jt] = u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
}

// Softmax and PV of one 32-key step for all row tiles of a wave, from its
// raw scores s.  Keys > lim[nr] (the lane's row position) are masked unless
// the whole step lies at or before kfull, the wave's first row position; V
// values of keys at or past kend are zeroed.
// c = scale * log2(e) > 0 (the host rejects other scales), so the row max of
// c*s is c times the max of s.
template <int D>
__device__ inline void step_softmax_pv(const f32x4 (&s)[kRowTiles][2], u32x4 (&av)[D / 16],
                                       PfAcc<D> (&a)[kRowTiles], int base, int kend, int kfull,
                                       const int (&lim)[kRowTiles], float c, int q4) {
  constexpr int kVd = D / 16;
  if (base + 32 > kend) {  // zero the V values of keys past the wave's last key
    uint32_t keep[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tok = base + 16 * (u >> 1) + 4 * q4 + 2 * (u & 1);
      keep[u] = (tok < kend ? 0x0000FFFFu : 0u) | (tok + 1 < kend ? 0xFFFF0000u : 0u);
    }
#pragma unroll
    for (int jt = 0; jt < kVd; ++jt)
#pragma unroll
      for (int u = 0; u < 4; ++u) av[jt][u] &= keep[u];
  }
  const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
  for (int nr = 0; nr < kRowTiles; ++nr) {
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] = s[nr][e >> 2][e & 3];
    if (base + 31 > kfull) {  // wave-uniform: some row does not see the whole step
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = base + 16 * (e >> 2) + 4 * q4 + (e & 3);
        sv[e] = tok <= lim[nr] ? sv[e] : -INFINITY;
      }
    }
    float mr = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) mr = fmaxf(mr, sv[e]);
    const float mx = row_max4(mr) * c;
    if (__builtin_amdgcn_ballot_w64(mx > a[nr].m + kSlack) != 0) {  // wave-uniform
      const float m_new = fmaxf(a[nr].m, mx);
      const float keep = __builtin_amdgcn_exp2f(a[nr].m - m_new);  // 0 on the first step
#pragma unroll
      for (int jt = 0; jt < kVd; ++jt) a[nr].o[jt] *= keep;
      a[nr].l *= keep;
      a[nr].m = m_new;
    }
    const float nm = -a[nr].m;
    u32x4 pb;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      pb[u] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(sv[2 * u], c, nm)),
                        __builtin_amdgcn_exp2f(fmaf(sv[2 * u + 1], c, nm)));
    a[nr].l = mma(ones, pb, a[nr].l);
#pragma unroll
    for (int jt = 0; jt < kVd; ++jt) a[nr].o[jt] = mma(av[jt], pb, a[nr].o[jt]);
  }
}

// The K and V tiles of one 32-key step, staged by the whole work-group:
// thread t holds parts t, t + kPfThreads, ... of the step's 2*32 rows (K rows
// first), 16 bytes each.  A part keeps its row, column and K|V role from step
// to step, so its byte offsets inside the block tile and inside the LDS tile
// are fixed per thread (StagePlan); a step only adds the two 16-token tiles'
// block offsets.  Keys past the sequence re-read its last live block (masked
// later); a table entry outside the pool sets `bad` (work-group uniform) and
// reads block 0 instead.
template <int D>
struct Stage {
  u32x4 part[kStageParts<D>];
};

template <int D>
struct StagePlan {
  const char* src[kStageParts<D>];   // K or V base + row-in-tile and column offset
  uint32_t lds[kStageParts<D>];      // byte offset in an LDS tile
  bool hi[kStageParts<D>];           // the part's row is in the step's second 16-token tile
};

template <int D>
__device__ inline StagePlan<D> stage_plan(const SeqView& c, int tid) {
  StagePlan<D> sp;
#pragma unroll
  for (int j = 0; j < kStageParts<D>; ++j) {
    const int idx = tid + kPfThreads * j;
    const int kv = idx / (32 * kRowParts<D>);
    const int rem = idx - kv * 32 * kRowParts<D>;
    const int row = rem / kRowParts<D>;
    const int col = rem - row * kRowParts<D>;
    sp.src[j] = (kv ? c.vbase : c.kbase) + (row & 15) * (D * 2) + col * 16;
    sp.lds[j] = (uint32_t)((kv * 32 + row) * kKvStride<D> + col * 16);
    sp.hi[j] = row >= 16;
  }
  return sp;
}

template <int D>
__device__ inline void stage_load(Stage<D>& st, const StagePlan<D>& sp, const SeqView& c,
                                  int base, bool& bad) {
  int64_t tile[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int tok0 = base + 16 * kt;
    const int lb = min(tok0 >> c.block_shift, c.nblocks_valid - 1);
    int phys = c.table[lb];
    if (phys < 0 || phys >= c.num_blocks) {
      bad = true;
      phys = 0;
    }
    tile[kt] = (int64_t)phys * c.block_stride + (int64_t)(tok0 & c.bmask) * (D * 2);
  }
#pragma unroll
  for (int j = 0; j < kStageParts<D>; ++j)
    st.part[j] = *(const u32x4*)(sp.src[j] + (sp.hi[j] ? tile[1] : tile[0]));
}

template <int D>
__device__ inline void stage_store(const Stage<D>& st, const StagePlan<D>& sp, unsigned char* buf) {
#pragma unroll
  for (int j = 0; j < kStageParts<D>; ++j) *(u32x4*)(buf + sp.lds[j]) = st.part[j];
}

// The work-group's walk over keys [kstart, kend_wg) in 32-key steps (kstart
// a multiple of 32): every thread stages its parts of the next step's K and V
// tiles from HBM while the waves compute the current one from LDS (two
// buffers, one barrier per step).  A wave takes the math of the steps below
// its own kend only; every wave stages and meets every barrier.
template <int D>
__device__ inline void attend_keys(PfAcc<D> (&a)[kRowTiles], const SeqView& c,
                                   const u32x4 (&qb)[kRowTiles][D / 32],
                                   const int (&lim)[kRowTiles], int kstart, int kend_wg, int kend,
                                   int kfull, float scale_log2, bool& bad,
                                   unsigned char (*sm_kv)[2 * 32 * kKvStride<D>], int tid, int r16,
                                   int q4) {
  const StagePlan<D> sp = stage_plan<D>(c, tid);
  Stage<D> st;
  stage_load<D>(st, sp, c, kstart, bad);
  stage_store<D>(st, sp, sm_kv[0]);
  __syncthreads();
  int buf = 0;
  for (int base = kstart; base < kend_wg; base += 32) {
    const bool more = base + 32 < kend_wg;
    if (more) stage_load<D>(st, sp, c, base + 32, bad);  // in flight during the math
    if (base < kend) {
      f32x4 s[kRowTiles][2];
      step_scores<D>(s, sm_kv[buf], qb, r16, q4);
      u32x4 av[D / 16];
      read_v<D>(av, sm_kv[buf] + 32 * kKvStride<D>, r16, q4);
      step_softmax_pv<D>(s, av, a, base, kend, kfull, lim, scale_log2, q4);
    }
    if (more) stage_store<D>(st, sp, sm_kv[buf ^ 1]);
    __syncthreads();
    buf ^= 1;
  }
}

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

  // Q^T operands of the lane's row in each tile (zero past the chunk) and the
  // causal limit of that row.
  u32x4 qb[kRowTiles][D / 32];
  int lim[kRowTiles];
#pragma unroll
  for (int nr = 0; nr < kRowTiles; ++nr) {
    const int row = wrow0 + 16 * nr + r16;
    const int qi = i0 + row / G;
    const int g = row - (row / G) * G;
    const bool valid = qi < nq;
    lim[nr] = valid ? pos0 + qi : 0;
    const char* qrow =
        (const char*)p.q + ((int64_t)(q0 + qi) * row_stride + head0 + (int64_t)g * D) * 2 + q4 * 16;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
      qb[nr][i] = valid ? *(const u32x4*)(qrow + 64 * i) : u32x4{0u, 0u, 0u, 0u};
  }

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
  }
  bool bad = false;
  // The key loop of attend_keys, written out.
  __shared__ __attribute__((aligned(16))) unsigned char sm_kv[2][2 * 32 * kKvStride<D>];
  {
    const StagePlan<D> sp = stage_plan<D>(c, tid);
    Stage<D> st;
    stage_load<D>(st, sp, c, 0, bad);
    stage_store<D>(st, sp, sm_kv[0]);
    __syncthreads();
    int buf = 0;
    for (int base = 0; base < kend_wg; base += 32) {
      const bool more = base + 32 < kend_wg;
      if (more) stage_load<D>(st, sp, c, base + 32, bad);  // in flight during the math
      if (base < kend) {
        f32x4 s[kRowTiles][2];
        step_scores<D>(s, sm_kv[buf], qb, r16, q4);
        u32x4 av[D / 16];
        read_v<D>(av, sm_kv[buf] + 32 * kKvStride<D>, r16, q4);
        step_softmax_pv<D>(s, av, a, base, kend, kfull, lim, p.scale_log2, q4);
      }
      if (more) stage_store<D>(st, sp, sm_kv[buf ^ 1]);
      __syncthreads();
      buf ^= 1;
    }
  }
  if (!wave_rows) return;

#pragma unroll
  for (int nr = 0; nr < kRowTiles; ++nr) {
    const int row = wrow0 + 16 * nr + r16;
    const int qi = i0 + row / G;
    const int g = row - (row / G) * G;
    if (qi >= nq) continue;
    const float inv = bad ? __builtin_nanf("") : 1.0f / a[nr].l[0];
    // o[jt][rr] is head dim 16 jt + 4 q4 + rr of the lane's row
    uint16_t* orow = out + (int64_t)(q0 + qi) * row_stride + head0 + (int64_t)g * D + 4 * q4;
#pragma unroll
    for (int jt = 0; jt < kVd; ++jt) {
      const f32x4 o = a[nr].o[jt];
      *(u32x2*)(orow + 16 * jt) = u32x2{pack_bf16(o[0] * inv, o[1] * inv),
                                        pack_bf16(o[2] * inv, o[3] * inv)};
    }
  }
}

// Shared-prefix decode, prefix part: the decode queries of every member of a
// group (sequences whose tables start with the same physical blocks) attend
// the group's shared keys once per work-group instead of once per sequence
// ("How PagedAttention works", section "A strong answer": one set of prefix
// blocks with N tables pointing at it).  Rows are (member, query head) pairs
// of one KV head, 128 per work-group, over one partition of the prefix keys;
// no causal limit applies, since every member's position is past its prefix.
// The result is a partial (unnormalised O, reference max m, sum l) in
// workspace slot `partition` of the row, merged with the tail partials by
// prefix_merge.
//
// Work order: group g owns work-groups wg_start[g] ..; inside it, all member
// tiles of one (partition, KV head) pair run on one XCD (work-group x runs on
// XCD x % 8), so the pair's K/V tiles stay in that XCD's L2.
template <int D>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void prefix_attend_kernel(DecodeParams p) {
  constexpr int kVd = D / 16;
  const PrefixGroups& pg = p.prefix;
  const int x = blockIdx.x;
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
  const int kend_wg = min(tokens, kstart + pg.partition);

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

  u32x4 qb[kRowTiles][D / 32];
  int lim[kRowTiles];
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
  }
  bool bad = false;
  __shared__ __attribute__((aligned(16))) unsigned char sm_kv[2][2 * 32 * kKvStride<D>];
  attend_keys<D>(a, c, qb, lim, kstart, kend_wg, kend, kfull, p.scale_log2, bad, sm_kv, tid,
                 r16, q4);
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

hipError_t launch_prefix_attend(const DecodeParams& p, int head_dim, hipStream_t stream) {
  const int wgs = p.prefix.wg_start[p.prefix.num_groups];
  if (wgs <= 0) return hipSuccess;
  const dim3 block(kPfWaves * 64);
  if (head_dim == 128)
    prefix_attend_kernel<128><<<dim3(wgs), block, 0, stream>>>(p);
  else if (head_dim == 64)
    prefix_attend_kernel<64><<<dim3(wgs), block, 0, stream>>>(p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
