// Paged decode attention on the vector ALUs (fp32 or bf16 storage, fp32 math).
//
// One 64-lane work-group per (sequence, KV head, partition).  A token's
// head_dim-long K/V row is split over LPT lanes, each holding one 16-byte
// vector (4 fp32 or 8 bf16 values), so one wave works on TPW = 64/LPT tokens
// at a time, one per lane group.  Each lane group runs its own online softmax
// over the tokens it visits (running max m, running sum l, unnormalised
// output acc for its slice of head_dim, for every query head of the GQA
// group); the groups are merged at the end with a butterfly.
//
// Scores are kept in base-2 units (q.k * scale * log2 e) so every exponential
// is a single exp2.
//
// The gather: position t of the sequence sits in logical block t / block_size
// at slot t % block_size, and the block table gives the physical block
// (lihaoran.work PagedAttention explainer, section "A block table maps logical
// order to physical storage").  Tokens of the partition past the sequence end
// are never loaded, so NaN left in unused slots is never touched.
#include <math.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool BF16>
struct Vec16;

template <>
struct Vec16<false> {  // fp32: 4 values per 16 bytes
  static constexpr int kN = 4;
  __device__ static void unpack(const u32x4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static void store(void* base, int64_t idx, float x) {
    ((float*)base)[idx] = x;
  }
};

template <>
struct Vec16<true> {  // bf16: 8 values per 16 bytes
  static constexpr int kN = 8;
  __device__ static void unpack(const u32x4& v, float* f) {
    f[0] = bf16_lo(v.x);
    f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y);
    f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z);
    f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w);
    f[7] = bf16_hi(v.w);
  }
  __device__ static void store(void* base, int64_t idx, float x) {
    ((uint16_t*)base)[idx] = f32_to_bf16(x);
  }
};

template <bool BF16, int D, int G>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeParams p) {
  using V = Vec16<BF16>;
  constexpr int kVec = V::kN;        // values per lane per row
  constexpr int kLpt = D / kVec;     // lanes per token row
  constexpr int kTpw = 64 / kLpt;    // tokens per wave step
  constexpr int kElem = BF16 ? 2 : 4;
  static_assert(kLpt >= 1 && kLpt <= 64 && (64 % kLpt) == 0, "row must tile the wave");

  const WorkItem w = decode_work_item(p, blockIdx.x);
  const int lane = threadIdx.x;
  const int sub = lane % kLpt;       // which 16-byte slice of the row
  const int grp = lane / kLpt;       // which token stream
  const int len = p.seq_lens[w.seq];
  const int64_t out_row0 = (int64_t)w.seq * p.num_heads + (int64_t)w.head * G;

  if (!seq_len_ok(p, len) || len == 0) {
    if (w.part == 0) store_new_token(p, w.seq, w.head, D * kElem, lane);
    if (w.part == 0 && grp == 0) {
      const float fill = len == 0 ? 0.0f : __builtin_nanf("");
      for (int g = 0; g < G; ++g)
        for (int e = 0; e < kVec; ++e) V::store(p.out, (out_row0 + g) * D + sub * kVec + e, fill);
    }
    return;
  }
  const int pstart = w.part * p.partition_size;
  if (pstart >= len) return;
  const int pend = range_end(pstart, p.partition_size, len);
  const int nparts = ceil_div_i(len, p.partition_size);

  float qf[G][kVec];
  for (int g = 0; g < G; ++g) {
    const u32x4 raw =
        *(const u32x4*)((const char*)p.q + ((out_row0 + g) * D + sub * kVec) * kElem);
    V::unpack(raw, qf[g]);
  }

  const NewToken nt = new_token(p, w.seq, w.head, len, D * kElem);
  float m[G], l[G], acc[G][kVec];
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
    for (int e = 0; e < kVec; ++e) acc[g][e] = 0.0f;
  }
  bool bad = false;

  const int32_t* table = p.block_tables + (int64_t)w.seq * p.max_blocks_per_seq;
  const int bmask = p.block_size - 1;
  for (int t = pstart + grp; t < pend; t += kTpw) {
    int phys = table[t >> p.block_shift];
    if (phys < 0 || phys >= p.num_blocks) {  // corrupt table entry: poison, never read it
      bad = true;
      phys = 0;
    }
    const int64_t row = ((((int64_t)phys * p.kv_heads + w.head) << p.block_shift) + (t & bmask));
    const int64_t byte_off = (row * D + sub * kVec) * kElem;
    const bool fresh = t == nt.pos;  // fused append: the new token comes from its buffer
    const char* kp = fresh ? nt.krow + sub * kVec * kElem : (const char*)p.k_cache + byte_off;
    const char* vp = fresh ? nt.vrow + sub * kVec * kElem : (const char*)p.v_cache + byte_off;
    float kf[kVec], vf[kVec];
    V::unpack(*(const u32x4*)kp, kf);
    V::unpack(*(const u32x4*)vp, vf);
    for (int g = 0; g < G; ++g) {
      float dot = 0.0f;
      for (int e = 0; e < kVec; ++e) dot = fmaf(qf[g][e], kf[e], dot);
      for (int o = 1; o < kLpt; o <<= 1) dot += __shfl_xor(dot, o);
      const float sc = dot * p.scale_log2;
      const float mn = fmaxf(m[g], sc);
      const float keep = exp2f(m[g] - mn);  // 0 on the group's first token
      const float pe = exp2f(sc - mn);
      l[g] = l[g] * keep + pe;
      for (int e = 0; e < kVec; ++e) acc[g][e] = fmaf(pe, vf[e], acc[g][e] * keep);
      m[g] = mn;
    }
  }
  if (bad) {
    for (int g = 0; g < G; ++g) {
      l[g] = __builtin_nanf("");
      for (int e = 0; e < kVec; ++e) acc[g][e] = __builtin_nanf("");
    }
  }

  // Merge the kTpw token streams: pairwise (m, l, acc) combination.
  for (int o = kLpt; o < 64; o <<= 1) {
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], o);
      const float lo = __shfl_xor(l[g], o);
      const float mn = fmaxf(m[g], mo);
      const float a = m[g] == -INFINITY ? 0.0f : exp2f(m[g] - mn);
      const float b = mo == -INFINITY ? 0.0f : exp2f(mo - mn);
      l[g] = l[g] * a + lo * b;
      for (int e = 0; e < kVec; ++e) {
        const float ao = __shfl_xor(acc[g][e], o);
        acc[g][e] = acc[g][e] * a + ao * b;
      }
      m[g] = mn;
    }
  }

  // fused append: the cache write comes after every cache read of this group
  if (w.part == 0) store_new_token(p, w.seq, w.head, D * kElem, lane);
  if (grp != 0) return;
  if (nparts == 1) {
    for (int g = 0; g < G; ++g) {
      const float inv = 1.0f / l[g];
      for (int e = 0; e < kVec; ++e)
        V::store(p.out, (out_row0 + g) * D + sub * kVec + e, acc[g][e] * inv);
    }
  } else {
    for (int g = 0; g < G; ++g) {
      const int64_t slot = (out_row0 + g) * p.num_partitions + w.part;
      for (int e = 0; e < kVec; ++e) p.ws_o[slot * D + sub * kVec + e] = acc[g][e];
      if (sub == 0) {
        p.ws_ml[slot * 2 + 0] = m[g];
        p.ws_ml[slot * 2 + 1] = l[g];
      }
    }
  }
}

template <bool BF16, int D>
hipError_t launch_g(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.num_partitions * p.num_seqs * p.kv_heads));
  switch (p.group) {
    case 1: decode_valu_kernel<BF16, D, 1><<<grid, 64, 0, stream>>>(p); break;
    case 2: decode_valu_kernel<BF16, D, 2><<<grid, 64, 0, stream>>>(p); break;
    case 4: decode_valu_kernel<BF16, D, 4><<<grid, 64, 0, stream>>>(p); break;
    case 8: decode_valu_kernel<BF16, D, 8><<<grid, 64, 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_valu(const DecodeParams& p, bool is_bf16, int head_dim,
                              hipStream_t stream) {
  if (is_bf16) {
    if (head_dim == 64) return launch_g<true, 64>(p, stream);
    if (head_dim == 128) return launch_g<true, 128>(p, stream);
  } else {
    if (head_dim == 64) return launch_g<false, 64>(p, stream);
    if (head_dim == 128) return launch_g<false, 128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
