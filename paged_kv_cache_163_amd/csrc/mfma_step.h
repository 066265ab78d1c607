// One wave's 32-token step of paged decode attention on the gfx950 matrix
// cores, shared by the split-partition decode work-group and the shared-prefix
// tail work-groups.
//
// A step is two 16-token tiles.  Block sizes are powers of two >= 16, so a
// tile never straddles two physical blocks and costs one block-table read
// (lihaoran.work PagedAttention explainer, section "A block table maps
// logical order to physical storage": logical block t / block_size, slot
// t % block_size).
//
// Both contractions run on v_mfma_f32_16x16x32_bf16.  Operand layout (lane
// l = 16*q4 + r16): A[i][k] sits in lane (i, k/8) as 8 bf16, B[k][j] in lane
// (j, k/8), and lane l ends with C[4*q4 + r][r16], r = 0..3.
//
//  * Scores.  S^T[token][g] = K[token][:] . Q[g][:] with A = the K tile (16
//    tokens x 32 head-dim values per instruction, head_dim/32 instructions)
//    and B = Q^T (the GQA group's query heads in columns 0..G-1, zero
//    columns above).  Lane (r16, q4) loads token r16, bytes [64*i + 16*q4,
//    +16) of the row for instruction i straight into the A operand.  Lane l
//    ends with the scores of query head g = r16 for tokens 4*q4 + r of each
//    tile, so the softmax needs no lane exchange except the max over the
//    four lanes sharing r16.
//  * Output.  O^T[d][g] += V^T[d][token] * P^T[token][g] over the step's 32
//    tokens.  B = P^T is built from the lane's own probabilities: element e
//    of lane (r16, q4) is token tau(q4, e) = 16*(e/4) + 4*q4 + e%4, exactly
//    the tokens whose scores the lane holds.  A = V^T needs 8 tokens of one
//    head-dim row per lane: each lane loads rows tau(q4, 0..7), column slice
//    [VD*r16, +VD) with VD = head_dim/16 (every V load instruction reads four
//    whole rows, fully coalesced), and transposes the 8 x VD block in
//    registers with byte permutes.  Row i of output tile jt is head
//    dimension VD*i + jt.
//
// Exponentials are v_exp_f32 (__builtin_amdgcn_exp2f): no denormal results,
// which only removes probabilities below 2^-126 that bf16 rounding keeps as
// denormals; measured ~0.6 % faster than the library exp2f on the 70B batch.
//
// Softmax per step in base-2 units: step max over the lane's 8 scores and
// its 3 partner lanes; (m, l, O) rescaled when the max rises; p =
// exp2(s - m) rounded to bf16 for the PV product and summed into l in that
// same rounded form, so the output is an exact convex combination of V rows
// up to fp32 accumulation.  Tokens at or past `pend` get score -inf and
// their V rows are zeroed by select (0 * NaN would poison the sum).
#pragma once

#include <math.h>

#include "pa_internal.h"

namespace pa {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

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
  u32x4 k[2][D / 32];           // A operands of the score MFMAs, per tile
  typename VRow<D>::T v[8];     // V rows tau(q4, e), e = 0..7
};

template <int D>
struct Acc {
  f32x4 o[D / 16];  // O^T tiles: o[jt][r] = O[g = r16][d = VD*(4*q4 + r) + jt]
  float m;          // running max (base-2 units), same in the 4 lanes of r16
  float l;          // this lane's share of the running sum
};

// Where one sequence's K/V live.
struct SeqView {
  const char* kbase;      // k_cache bytes + KV-head offset
  const char* vbase;
  const int32_t* table;   // the sequence's block-table row
  int64_t block_stride;   // bytes between physical blocks
  int nblocks_valid;      // ceil(len / block_size)
  int num_blocks;
  int block_shift;
  int bmask;
};

__device__ inline f32x4 mma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int D>
__device__ inline void reset(Acc<D>& a) {
#pragma unroll
  for (int jt = 0; jt < D / 16; ++jt) a.o[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  a.m = -INFINITY;
  a.l = 0.f;
}

// Issue the loads of the step starting at token `base` (a multiple of 32).
// Tiles wholly past the sequence re-read its last live block (masked later),
// so every load stays inside the caches.  A table entry outside the pool sets
// `bad` and reads block 0 instead.  Decode reads K/V once per launch, so by
// default (kStream) the loads are non-temporal: they do not displace reusable
// lines from L2/MALL (measured ~10 % faster on the 70B-shaped batch).
// Prefill re-reads every tile from several waves and work-groups and wants
// them cached (kStream = false).
template <typename T, bool kStream>
__device__ inline T load16(const T* p) {
  if constexpr (kStream)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <int D, bool kStream = true>
__device__ inline void load_step(StepRegs<D>& r, const SeqView& c, int base, int r16, int q4,
                                 bool& bad) {
  constexpr int kRow = D * 2;  // bytes per token row
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int tok0 = base + 16 * kt;
    const int lb = min(tok0 >> c.block_shift, c.nblocks_valid - 1);
    int phys = c.table[lb];
    if (phys < 0 || phys >= c.num_blocks) {
      bad = true;
      phys = 0;
    }
    // wave-uniform 64-bit base + 32-bit lane offset (scalar-base addressing)
    const int64_t tile = (int64_t)phys * c.block_stride + (int64_t)(tok0 & c.bmask) * kRow;
    const char* kt_base = c.kbase + tile;
    const char* vt_base = c.vbase + tile;
    const uint32_t koff = (uint32_t)(r16 * kRow + q4 * 16);
    const uint32_t voff = (uint32_t)((4 * q4) * kRow + r16 * (D / 16) * 2);
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
      r.k[kt][i] = load16<u32x4, kStream>((const u32x4*)(kt_base + (koff + 64u * i)));
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r.v[4 * kt + e] = load16<typename VRow<D>::T, kStream>(
          (const typename VRow<D>::T*)(vt_base + (voff + (uint32_t)(e * kRow))));
  }
}

// Scores, online softmax and PV for one loaded step; tokens >= pend masked
// (every step holds at least one token below pend: its first).
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
    for (int i = 0; i < kKi; ++i) s[kt] = mma(r.k[kt][i], qb[i], s[kt]);
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
  const float keep = __builtin_amdgcn_exp2f(a.m - m_new);  // 0 on the first step
  u32x4 pb;
  float psum = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t lo = f32_to_bf16(__builtin_amdgcn_exp2f(t[2 * u] - m_new));
    const uint32_t hi = f32_to_bf16(__builtin_amdgcn_exp2f(t[2 * u + 1] - m_new));
    pb[u] = lo | (hi << 16);
    psum += __uint_as_float(lo << 16) + __uint_as_float(hi << 16);
  }
  a.l = a.l * keep + psum;
  a.m = m_new;
#pragma unroll
  for (int jt = 0; jt < kVd; ++jt) a.o[jt] *= keep;

  if (base + 32 > pend) {  // tail step: zero V rows past the end
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
      // v_perm_b32: bytes 0-3 select from the second operand, 4-7 from the first
      const uint32_t lo = r.v[2 * u][jt >> 1];
      const uint32_t hi = r.v[2 * u + 1][jt >> 1];
      av[u] = (jt & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                       : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
    a.o[jt] = mma(av, pb, a.o[jt]);
  }
}

// Fused append: in a loaded step, replace the operands of the token at
// offset `off` (0..31) of the step by that token's new K and V rows, staged
// in `sm` (the K row, then the V row; LDS that only the calling wave writes):
// K row 16*kt + r16 at bytes 64*i + 16*q4 (load_step), V row 16*(e/4) +
// 4*q4 + e%4 at bytes (D/16)*2*r16.  The step's math is then that of the
// appended cache.
template <int D>
__device__ inline void patch_new_token(StepRegs<D>& r, const unsigned char* sm, int off, int r16,
                                       int q4) {
  using VT = typename VRow<D>::T;
  const int kt_new = off >> 4;
  const int rr = off & 15;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    if (kt == kt_new) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) {
        const u32x4 v = *(const u32x4*)(sm + 64 * i + 16 * q4);
        r.k[kt][i] = r16 == rr ? v : r.k[kt][i];
      }
    }
  }
  const int e_new = 4 * kt_new + (rr & 3);
  const VT v = *(const VT*)(sm + D * 2 + (D / 16) * 2 * r16);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (e == e_new) r.v[e] = q4 == (rr >> 2) ? v : r.v[e];
}

// Finish a wave's running sum (the four lanes of each r16 hold shares).
template <int D>
__device__ inline void finish_wave(Acc<D>& a, bool bad) {
  a.l += __shfl_xor(a.l, 16);
  a.l += __shfl_xor(a.l, 32);
  if (bad) {
    a.l = __builtin_nanf("");
#pragma unroll
    for (int jt = 0; jt < D / 16; ++jt) a.o[jt] = f32x4{a.l, a.l, a.l, a.l};
  }
}

// Column of head dim d of query-head row g in a merge buffer.  Rows are D
// floats apart, so the 16 rows' lanes that write one head dim would share an
// LDS bank; XOR-ing the column with 4 g spreads them over the banks, and
// keeps every aligned group of four columns together (16-byte reads stay
// whole).  Measured before the swizzle: 1.8 M bank-conflict cycles per launch
// on the 70B-shaped batch.
template <int D>
__device__ inline int stash_col(int g, int d) {
  return d ^ ((4 * g) & (D - 1));
}

// Write one wave's (m, l, O) for query heads g < G into the merge buffers.
template <int D, int NW>
__device__ inline void stash_wave(const Acc<D>& a, float (*sm_o)[16][D], float (*sm_m)[16],
                                  float (*sm_l)[16], int wave, int r16, int q4, int G) {
  constexpr int kVd = D / 16;
  if (r16 < G) {
#pragma unroll
    for (int jt = 0; jt < kVd; ++jt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        sm_o[wave][r16][stash_col<D>(r16, kVd * (4 * q4 + rr) + jt)] = a.o[jt][rr];
    if (q4 == 0) {
      sm_m[wave][r16] = a.m;
      sm_l[wave][r16] = a.l;
    }
  }
}

// Merge the NW waves' stashes for element (g, d): returns (max, sum, output).
template <int D, int NW>
__device__ inline void merge_waves(const float (*sm_o)[16][D], const float (*sm_m)[16],
                                   const float (*sm_l)[16], int g, int d, float& mx, float& l,
                                   float& o) {
  mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < NW; ++v) mx = fmaxf(mx, sm_m[v][g]);
  o = 0.f;
  l = 0.f;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const float mv = sm_m[v][g];
    const float wt = mv == -INFINITY ? 0.f : exp2f(mv - mx);
    o += wt * sm_o[v][g][stash_col<D>(g, d)];
    l += wt * sm_l[v][g];
  }
}

}  // namespace mfma
}  // namespace pa
