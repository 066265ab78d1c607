// Persistent, load-balanced paged decode on the gfx950 matrix cores (bf16
// storage, fp32 accumulation).
//
// Why.  Decode batches mix sequence lengths, and every (sequence, KV head)
// pair is a different amount of work.  One work-group per pair leaves the
// GPU half idle at the end of the launch, and each work-group start pays a
// dependent-latency chain (length -> block table -> K/V) before its first
// byte arrives.  Here a fixed grid of work-groups (a few per compute unit)
// splits the total work evenly instead, and each work-group streams through
// its share without restarting.
//
// Work space.  Every (KV head h, sequence s) pair is a unit of
// n_s = ceil(len_s / 32) steps (mfma_step.h); units are laid out head-major
// (u = h*B + s), so global step x of unit (h, s) is h*S + prefix_s + k,
// S = sum_s n_s.  With T = Hkv*S total steps and N work-groups, work-group i
// takes steps [floor(i*T/N), floor((i+1)*T/N)).  Its share is a run of
// segments: whole units, plus possibly the tail of the unit it starts in and
// the head of the unit it ends in.  The hardware hands consecutive
// work-group ids to the 8 XCDs in turn, so id b is given share
// (b % 8) * N/8 + b / 8: each XCD walks one contiguous eighth of the
// head-major space, about one KV head when Hkv = 8, and its L2 keeps that
// head's shared-prefix blocks.
//
// Inside a work-group the waves interleave the steps of the current segment
// (wave w takes steps a + w, a + w + 4, ...).  Each wave's loads run one step
// ahead of its math across segment boundaries, so the next segment's first
// K/V tiles are in flight while the group merges the finished one.
//
// Segment end.  The waves merge (m, l, O) through LDS.  A whole unit writes
// its normalised bf16 output.  A cut unit writes its partial (m, l,
// unnormalised O) to the work-group's slot in the workspace and takes a
// ticket; the last of the unit's work-groups to arrive merges all partials
// and writes the output (same formula as decode_reduce.hip).  Tickets carry
// the call's epoch in their upper 32 bits, so stale values from earlier
// calls count as zero and the workspace needs no clearing.  Nothing waits
// on another work-group.
//
// Sequences of length 0 (zero rows) and lengths the table cannot serve (NaN
// rows) take no steps; work-group i writes those outputs for s = i, i+N, ...
#include "mfma_step.h"

namespace pa {
namespace {

using namespace mfma;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kXcds = 8;

__device__ inline int unit_steps(const DecodeParams& p, int len) {
  return (len > 0 && seq_len_ok(p, len)) ? (len + 31) >> 5 : 0;
}

__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// A run of steps of one unit inside this work-group's share (s < 0: none).
// Global step indices fit in int32: the host only picks this kernel when
// kv_heads * num_seqs * ceil(max_seq_len / 32) < 2^31.
struct Seg {
  int s, h, len;  // sequence, KV head, its length in tokens
  int a, b;       // local step range [a, b) covered here
  int ustart;     // global index of the unit's step 0 (identifies the segment)
};

__device__ inline int steps_of(int len) { return (len + 31) >> 5; }

// The segment after `c` within a share ending at global step `hi`.
__device__ inline Seg next_seg(const DecodeParams& p, const Seg& c, int hi) {
  Seg n;
  n.s = -1;
  n.ustart = c.ustart + steps_of(c.len);
  if (n.ustart >= hi) return n;
  int s = c.s, h = c.h;
  while (true) {  // skip sequences with no steps; ustart < hi guarantees a unit ahead
    if (++s == p.num_seqs) {
      s = 0;
      if (++h == p.kv_heads) return n;
    }
    const int len = uniform(p.seq_lens[s]);
    if (unit_steps(p, len) > 0) {
      n.s = s;
      n.h = h;
      n.len = len;
      break;
    }
  }
  n.a = 0;
  n.b = min(steps_of(n.len), hi - n.ustart);
  return n;
}

// One wave's position: local step k of segment seg (seg.s < 0: done).
struct Item {
  Seg seg;
  int k;
};

__device__ inline Item settle(const DecodeParams& p, Seg seg, int k, int wave, int hi) {
  while (seg.s >= 0 && k >= seg.b) {
    seg = next_seg(p, seg, hi);
    k = seg.a + wave;
  }
  Item it;
  it.seg = seg;
  it.k = k;
  return it;
}

template <int D>
struct Buf {
  StepRegs<D> r;
  bool bad;
};

template <int D>
__device__ inline void load_item(Buf<D>& buf, const DecodeParams& p, const Item& it, int r16,
                                 int q4) {
  const int64_t head_stride = (int64_t)p.block_size * D * 2;
  SeqView c;
  c.kbase = (const char*)p.k_cache + (int64_t)it.seg.h * head_stride;
  c.vbase = (const char*)p.v_cache + (int64_t)it.seg.h * head_stride;
  c.table = p.block_tables + (int64_t)it.seg.s * p.max_blocks_per_seq;
  c.block_stride = (int64_t)p.kv_heads * head_stride;
  c.nblocks_valid = (it.seg.len + p.block_size - 1) >> p.block_shift;
  c.num_blocks = p.num_blocks;
  c.block_shift = p.block_shift;
  c.bmask = p.block_size - 1;
  buf.bad = false;
  load_step<D>(buf.r, c, it.k * 32, r16, q4, buf.bad);
}

// Arrival count at this call's epoch, before this arrival.  Lock-free: a
// failed compare-and-swap means another arrival succeeded.
__device__ inline uint32_t ticket_arrive(uint64_t* t, uint32_t epoch) {
  unsigned long long cur = __hip_atomic_load((unsigned long long*)t, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
  while (true) {
    const uint32_t cnt = (uint32_t)(cur >> 32) == epoch ? (uint32_t)cur : 0u;
    const unsigned long long want = ((unsigned long long)epoch << 32) | (cnt + 1u);
    const unsigned long long prev = atomicCAS((unsigned long long*)t, cur, want);
    if (prev == cur) return cnt;
    cur = prev;
  }
}

// Index of the work-group whose share holds global step x.
__device__ inline int share_of(int64_t x, int64_t T, int64_t N) {
  return (int)(((x + 1) * N + T - 1) / T - 1);
}

// Two resident work-groups per compute unit: at most 256 registers per lane.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_stream_kernel(DecodeParams p) {
  constexpr int kKi = D / 32;
  constexpr int kQRow = D * 2 + 16;  // padded LDS row of one query head
  __shared__ float sm_o[kWaves][16][D];
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];
  __shared__ __attribute__((aligned(16))) unsigned char sm_q[16 * kQRow];
  __shared__ int64_t sm_scan[kWaves];
  __shared__ int64_t sm_find[2];
  __shared__ int sm_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int r16 = lane & 15;
  const int q4 = lane >> 4;
  const int B = p.num_seqs;
  const int G = p.group;
  const int Hq = p.num_heads;
  const int N = p.num_workgroups;
  uint16_t* out = (uint16_t*)p.out;

  // -- outputs of sequences that take no steps ------------------------------
  for (int s = blockIdx.x; s < B; s += N) {
    const int len = uniform(p.seq_lens[s]);
    if (unit_steps(p, len) == 0) {
      const uint16_t fill = len == 0 ? (uint16_t)0 : (uint16_t)0x7FC0;
      for (int i = tid; i < Hq * D; i += kThreads) out[(int64_t)s * Hq * D + i] = fill;
    }
  }

  // -- steps per KV head: S = sum_s n_s (block scan over the sequences) ------
  const int per = (B + kThreads - 1) / kThreads;
  const int s_begin = min(B, tid * per);
  const int s_end = min(B, s_begin + per);
  int64_t mine = 0;
  for (int s = s_begin; s < s_end; ++s) mine += unit_steps(p, p.seq_lens[s]);
  int64_t incl = mine;
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) sm_scan[wave] = incl;
  __syncthreads();
  int64_t before = incl - mine;
  int64_t S = 0;
  for (int v = 0; v < kWaves; ++v) {
    const int64_t t = sm_scan[v];
    if (v < wave) before += t;
    S += t;
  }
  S = uniform64(S);
  const int64_t T = S * p.kv_heads;
  const int64_t Neff = min((int64_t)N, T);
  const int bx = blockIdx.x;
  const int share = (N % kXcds == 0) ? (bx % kXcds) * (N / kXcds) + bx / kXcds : bx;
  if (share >= Neff) return;
  const int lo = (int)(share * T / Neff);
  const int hi = (int)((share + 1) * T / Neff);

  // -- locate the unit holding step lo ---------------------------------------
  const int h0 = (int)(lo / S);
  const int64_t x0 = lo - h0 * S;
  if (x0 >= before && x0 < before + mine) {
    int64_t at = before;
    for (int s = s_begin; s < s_end; ++s) {
      const int st = unit_steps(p, p.seq_lens[s]);
      if (x0 < at + st) {
        sm_find[0] = s;
        sm_find[1] = at;
        break;
      }
      at += st;
    }
  }
  __syncthreads();
  Seg seg0;
  seg0.h = h0;
  seg0.s = uniform((int)sm_find[0]);
  seg0.len = uniform(p.seq_lens[seg0.s]);
  seg0.ustart = (int)(h0 * S) + uniform((int)sm_find[1]);
  seg0.a = lo - seg0.ustart;
  seg0.b = min(steps_of(seg0.len), hi - seg0.ustart);

  // -- Q of a segment into LDS (16 bytes per thread) -------------------------
  const int qchunks = G * D / 8;
  auto q_src = [&](const Seg& sg) -> const u32x4* {
    const int g = tid / (D / 8);
    const int c = tid - g * (D / 8);
    return (const u32x4*)((const char*)p.q +
                          (((int64_t)sg.s * Hq + (int64_t)sg.h * G + g) * D) * 2 + c * 16);
  };
  auto q_dst = [&]() -> u32x4* {
    const int g = tid / (D / 8);
    const int c = tid - g * (D / 8);
    return (u32x4*)(sm_q + g * kQRow + c * 16);
  };
  if (tid < qchunks) *q_dst() = *q_src(seg0);
  __syncthreads();

  // -- stream ---------------------------------------------------------------
  // Each wave walks its items (segment, step) with loads one item ahead; the
  // two register sets keep fixed roles (A-half / B-half of the loop).  Before
  // an item of a later segment is computed, every segment up to it is
  // finished: waves merge through LDS, the output or partial is written, and
  // the next segment's Q (prefetched into registers) moves into LDS.  All
  // waves finish the same segments in the same order.
  Buf<D> bufA, bufB;
  Item cur = settle(p, seg0, seg0.a + wave, wave, hi);
  if (cur.seg.s >= 0) load_item<D>(bufA, p, cur, r16, q4);
  Seg ms = seg0;
  Acc<D> acc;
  reset(acc);
  bool segbad = false;
  u32x4 qnext = u32x4{0u, 0u, 0u, 0u};
  // The Q operand is re-read from LDS for every step (short-lived registers).
  auto read_q = [&](u32x4* qb) {
#pragma unroll
    for (int i = 0; i < kKi; ++i)
      qb[i] = r16 < G ? *(const volatile u32x4*)(sm_q + r16 * kQRow + 64 * i + 16 * q4)
                      : u32x4{0u, 0u, 0u, 0u};
  };
  auto begin_segment = [&]() {
    const Seg nseg = next_seg(p, ms, hi);
    if (nseg.s >= 0 && tid < qchunks) qnext = *q_src(nseg);
  };
  auto finish_segment = [&]() {
    finish_wave(acc, segbad);
    stash_wave<D, kWaves>(acc, sm_o, sm_m, sm_l, wave, r16, q4, G);
    __syncthreads();
    const Seg nseg = next_seg(p, ms, hi);
    if (nseg.s >= 0 && tid < qchunks) *q_dst() = qnext;  // every wave has read qb

    const int64_t row0 = (int64_t)ms.s * Hq + (int64_t)ms.h * G;
    const int ms_n = steps_of(ms.len);
    if (ms.a == 0 && ms.b == ms_n) {
      for (int i = tid; i < G * D; i += kThreads) {
        const int g = i / D;
        const int d = i - g * D;
        float mx, l, o;
        merge_waves<D, kWaves>(sm_o, sm_m, sm_l, g, d, mx, l, o);
        out[(row0 + g) * D + d] = f32_to_bf16(o / l);
      }
    } else {
      const int psz = G * (D + 2);
      float* slot = p.partials + ((int64_t)share * 2 + (ms.a > 0 ? 0 : 1)) * psz;
      for (int i = tid; i < G * D; i += kThreads) {
        const int g = i / D;
        const int d = i - g * D;
        float mx, l, o;
        merge_waves<D, kWaves>(sm_o, sm_m, sm_l, g, d, mx, l, o);
        slot[2 * G + i] = o;
        if (d == 0) {
          slot[g] = mx;
          slot[G + g] = l;
        }
      }
      __threadfence();
      __syncthreads();
      const int64_t U = ms.ustart;
      const int i0 = share_of(U, T, Neff);
      const int i1 = share_of(U + ms_n - 1, T, Neff);
      if (tid == 0) {
        const uint32_t earlier = ticket_arrive(p.tickets + (int64_t)ms.h * B + ms.s, p.epoch);
        sm_flag = (int)earlier + 1 == i1 - i0 + 1;
      }
      __syncthreads();
      if (sm_flag) {  // last part to arrive: merge every part of the unit
        __threadfence();
        for (int i = tid; i < G * D; i += kThreads) {
          const int g = i / D;
          float mx = -INFINITY;
          for (int w = i0; w <= i1; ++w) {
            const int64_t wlo = (int64_t)w * T / Neff;
            const float* ps = p.partials + ((int64_t)w * 2 + (wlo > U ? 0 : 1)) * psz;
            mx = fmaxf(mx, ps[g]);
          }
          float o = 0.f, l = 0.f;
          for (int w = i0; w <= i1; ++w) {
            const int64_t wlo = (int64_t)w * T / Neff;
            const float* ps = p.partials + ((int64_t)w * 2 + (wlo > U ? 0 : 1)) * psz;
            const float wt = exp2f(ps[g] - mx);
            o += wt * ps[2 * G + i];
            l += wt * ps[G + g];
          }
          out[(row0 + g) * D + (i - g * D)] = f32_to_bf16(o / l);
        }
      }
    }
    __syncthreads();  // merge buffers and sm_q are reused by the next segment
    ms = nseg;
    reset(acc);
    segbad = false;
  };
  // Finish segments until `cur` lies in `ms`; false once every segment is done.
  auto catch_up = [&]() -> bool {
    while (ms.s >= 0 && !(cur.seg.s >= 0 && cur.seg.ustart == ms.ustart)) {
      finish_segment();
      if (ms.s >= 0) begin_segment();
    }
    return ms.s >= 0;
  };
  begin_segment();
  while (true) {
    if (!catch_up()) break;
    {
      const Item nx = settle(p, cur.seg, cur.k + kWaves, wave, hi);
      if (nx.seg.s >= 0) load_item<D>(bufB, p, nx, r16, q4);
      u32x4 qb[kKi];
      read_q(qb);
      compute_step<D>(bufA.r, acc, qb, cur.k * 32, cur.seg.len, p.scale_log2, q4);
      segbad |= bufA.bad;
      cur = nx;
    }
    if (!catch_up()) break;
    {
      const Item nx = settle(p, cur.seg, cur.k + kWaves, wave, hi);
      if (nx.seg.s >= 0) load_item<D>(bufA, p, nx, r16, q4);
      u32x4 qb[kKi];
      read_q(qb);
      compute_step<D>(bufB.r, acc, qb, cur.k * 32, cur.seg.len, p.scale_log2, q4);
      segbad |= bufB.bad;
      cur = nx;
    }
  }
}

}  // namespace

hipError_t launch_decode_stream(const DecodeParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid((unsigned)p.num_workgroups);
  if (head_dim == 128)
    decode_stream_kernel<128><<<grid, kThreads, 0, stream>>>(p);
  else if (head_dim == 64)
    decode_stream_kernel<64><<<grid, kThreads, 0, stream>>>(p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
