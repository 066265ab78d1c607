// Paged decode attention on the gfx950 matrix cores (bf16 storage, fp32
// accumulation).
//
// Work decomposition.  One work-group of kWaves waves per (sequence, KV head,
// partition).  A partition is cut into 32-token steps; wave w of the group
// takes steps w, w + kWaves, ...  A step is two 16-token tiles.  Block sizes
// are powers of two >= 16, so a tile never straddles two physical blocks and
// costs one block-table read (lihaoran.work PagedAttention explainer, section
// "A block table maps logical order to physical storage": logical block
// t / block_size, slot t % block_size).
//
// Both contractions of a step run on v_mfma_f32_16x16x32_bf16.  Its operand
// layout (lane l = 16*q4 + r16): A[i][k] sits in lane (i, k/8) as 8 bf16,
// B[k][j] in lane (j, k/8), and lane l ends with C[4*q4 + r][r16], r = 0..3.
//
//  * Scores.  S^T[token][g] = K[token][:] . Q[g][:] with A = the K tile
//    (16 tokens x 32 head-dim values per instruction, head_dim/32
//    instructions) and B = Q^T (the GQA group's query heads in columns
//    0..G-1, zero columns above).  Each lane loads 16 bytes of one token's
//    row straight into the A operand: lane (r16, q4) reads token r16, bytes
//    [64*i + 16*q4, +16) for instruction i, so each load instruction covers
//    64 contiguous bytes of 16 rows.  Lane l's scores are for query head
//    g = r16 and tokens 4*q4 + r of each tile: every lane holds 8 scores of
//    ONE query head, so the softmax needs no lane exchange except the
//    max over the four lanes sharing r16.
//  * Output.  O^T[d][g] += V^T[d][token] * P^T[token][g], contraction over 32
//    tokens.  B = P^T comes from the lane's own probabilities: element e of
//    lane (r16, q4) is token tau(q4, e) = 16*(e/4) + 4*q4 + e%4, exactly the
//    tokens whose scores the lane holds.  A = V^T needs 8 tokens per lane for
//    one head-dim row, so each lane loads rows tau(q4, 0..7), its own
//    head_dim/16-wide column slice [VD*r16, +VD) -- every V load instruction
//    reads four whole rows, fully coalesced -- and transposes the 8 x VD
//    block in registers with byte permutes.  Row i of output tile jt is head
//    dimension VD*i + jt.
//
// Online softmax per step in base-2 units: the step max over the lane's 8
// scores and its 3 partner lanes, rescale (m, l, O) when it rises, p =
// exp2(s - m) rounded to bf16 for the PV product (accumulation stays fp32).
// Tokens at or past the partition end get score -inf and their V rows are
// zeroed by select before the product (0 * NaN would poison the sum).
//
// Loads are software-pipelined one step ahead (two register sets).
// At the end the waves of the group merge (m, l, O) through LDS; a
// single-partition sequence writes its normalised bf16 output directly,
// otherwise the partial goes to the workspace for the reduce kernel.
#include <math.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;

template <int D>
struct VRow;  // one lane's slice of a V row: D/16 bf16 values
template <>
struct VRow<128> {
  using T = u32x4;
};
template <>
struct VRow<64> {
  using T = u32x2;
};

template <int D>
struct StepRegs {
  static constexpr int kKi = D / 32;
  u32x4 k[2][kKi];                  // A operands of the score MFMAs, per tile
  typename VRow<D>::T v[8];         // V rows tau(q4, e), e = 0..7
};

__device__ inline f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Element jt of each of two packed-bf16 words, packed low/high into one word.
template <int JT>
__device__ inline uint32_t pick_pair(uint32_t lo_src, uint32_t hi_src) {
  // v_perm_b32: result byte i = byte sel_i of {hi_src:bytes 4-7, lo_src:bytes 0-3}
  return __builtin_amdgcn_perm(hi_src, lo_src, (JT & 1) ? 0x07060302u : 0x05040100u);
}

template <int D>
__device__ inline uint32_t vword(const typename VRow<D>::T& r, int i) {
  return r[i];
}

struct Ctx {
  const char* kbase;        // k_cache bytes
  const char* vbase;
  const int32_t* table;     // this sequence's block table
  int64_t head_stride;      // bytes between (block, head) tiles
  int64_t block_stride;     // bytes between physical blocks
  int nblocks_valid;        // ceil(len / block_size)
  int num_blocks;
  int block_shift;
  int bmask;
};

template <int D>
__device__ inline void load_step(StepRegs<D>& r, const Ctx& c, int base, int r16, int q4,
                                 bool& bad) {
  constexpr int kRow = D * 2;  // bytes per token row
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int tok0 = base + 16 * kt;
    int lb = tok0 >> c.block_shift;
    lb = min(lb, c.nblocks_valid - 1);  // tiles past the end re-read a live block (masked)
    int phys = c.table[lb];
    if (phys < 0 || phys >= c.num_blocks) {
      bad = true;
      phys = 0;
    }
    const int64_t tile = (int64_t)phys * c.block_stride + (int64_t)(tok0 & c.bmask) * kRow;
    const char* kp = c.kbase + tile + r16 * kRow + q4 * 16;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) r.k[kt][i] = *(const u32x4*)(kp + 64 * i);
    const char* vp = c.vbase + tile + (4 * q4) * kRow + r16 * (D / 16) * 2;
#pragma unroll
    for (int e = 0; e < 4; ++e) r.v[4 * kt + e] = *(const typename VRow<D>::T*)(vp + e * kRow);
  }
}

template <int D>
struct Acc {
  f32x4 o[D / 16];  // O^T tiles
  float m;
  float l;
};

template <int D>
__device__ inline void compute_step(StepRegs<D>& r, Acc<D>& a, const u32x4* qb, int base,
                                    int pend, float scale_log2, int q4) {
  constexpr int kKi = D / 32;
  constexpr int kVd = D / 16;
  f32x4 s[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kKi; ++i) s[kt] = mfma(r.k[kt][i], qb[i], s[kt]);
  }
  float t[8];
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int tok = base + 16 * (e >> 2) + 4 * q4 + (e & 3);
    const float v = s[e >> 2][e & 3] * scale_log2;
    t[e] = tok < pend ? v : -INFINITY;
    mx = fmaxf(mx, t[e]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(a.m, mx);
  const float keep = exp2f(a.m - m_new);  // 0 on the wave's first step
  float psum = 0.f;
  float pe[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pe[e] = exp2f(t[e] - m_new);
    psum += pe[e];
  }
  u32x4 pb;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    pb[u] = (uint32_t)f32_to_bf16(pe[2 * u]) | ((uint32_t)f32_to_bf16(pe[2 * u + 1]) << 16);
  a.l = a.l * keep + psum;
  a.m = m_new;
#pragma unroll
  for (int jt = 0; jt < kVd; ++jt) a.o[jt] *= keep;

  if (base + 32 > pend) {  // tail step: zero V rows past the partition end
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tok = base + 16 * (e >> 2) + 4 * q4 + (e & 3);
      if (tok >= pend) r.v[e] = typename VRow<D>::T{};
    }
  }
#pragma unroll
  for (int jt = 0; jt < kVd; ++jt) {
    u32x4 av;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t lo = r.v[2 * u][jt >> 1];
      const uint32_t hi = r.v[2 * u + 1][jt >> 1];
      av[u] = (jt & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                       : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
    a.o[jt] = mfma(av, pb, a.o[jt]);
  }
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) void decode_mfma_kernel(DecodeParams p) {
  constexpr int kKi = D / 32;
  constexpr int kVd = D / 16;
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

  Ctx c;
  c.kbase = (const char*)p.k_cache;
  c.vbase = (const char*)p.v_cache;
  c.table = p.block_tables + (int64_t)w.seq * p.max_blocks_per_seq;
  c.head_stride = (int64_t)p.block_size * D * 2;
  c.block_stride = (int64_t)p.kv_heads * c.head_stride;
  c.kbase += (int64_t)w.head * c.head_stride;
  c.vbase += (int64_t)w.head * c.head_stride;
  c.nblocks_valid = (len + p.block_size - 1) >> p.block_shift;
  c.num_blocks = p.num_blocks;
  c.block_shift = p.block_shift;
  c.bmask = p.block_size - 1;

  Acc<D> a;
#pragma unroll
  for (int jt = 0; jt < kVd; ++jt) a.o[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  a.m = -INFINITY;
  a.l = 0.f;
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
  a.l += __shfl_xor(a.l, 16);
  a.l += __shfl_xor(a.l, 32);
  if (bad) {
    a.l = __builtin_nanf("");
#pragma unroll
    for (int jt = 0; jt < kVd; ++jt) a.o[jt] = f32x4{a.l, a.l, a.l, a.l};
  }

  // Merge the waves of the group through LDS.
  if (r16 < G) {
#pragma unroll
    for (int jt = 0; jt < kVd; ++jt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sm_o[wave][r16][kVd * (4 * q4 + rr) + jt] = a.o[jt][rr];
    if (q4 == 0) {
      sm_m[wave][r16] = a.m;
      sm_l[wave][r16] = a.l;
    }
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kWaves * 64) {
    const int g = i / D;
    const int d = i - g * D;
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) mx = fmaxf(mx, sm_m[v][g]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float mv = sm_m[v][g];
      const float wt = mv == -INFINITY ? 0.f : exp2f(mv - mx);
      o += wt * sm_o[v][g][d];
      l += wt * sm_l[v][g];
    }
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
