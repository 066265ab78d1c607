// Paged attention on the vector ALUs (fp32 or bf16 storage, fp32 math): the
// decode kernel for every shape the matrix-core kernel does not take (fp32,
// block sizes below 16), and the chunked prefill for those shapes.
//
// One 64-lane work-group attends one query row per KV head at a time.  A
// token's head_dim-long K/V row is split over LPT lanes, each holding one
// 16-byte vector (4 fp32 or 8 bf16 values), so one wave works on TPW = 64/LPT
// tokens at a time, one per lane group.  Each lane group runs its own online
// softmax over the tokens it visits (running max m, running sum l,
// unnormalised output acc for its slice of head_dim, for every query head of
// the GQA group); the groups are merged at the end with a butterfly.
//
// Scores are kept in base-2 units (q.k * scale * log2 e) so every exponential
// is a single exp2.
//
// The gather: position t of the sequence sits in logical block t / block_size
// at slot t % block_size, and the block table gives the physical block
// (lihaoran.work PagedAttention explainer, section "A block table maps logical
// order to physical storage").  Tokens past the attended range are never
// loaded, so NaN left in unused slots is never touched.
//
// Decode: one work-group per (sequence, KV head, partition), layer =
// blockIdx.y over a layered pool.  Prefill: one work-group per (sequence, KV
// head, tile of kPrefillValuRows chunk queries); the query at position p
// attends positions [0, p] (the same explainer section: causal attention over
// the visible history).
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

// Where one (sequence, KV head)'s K/V live.
struct ValuView {
  const char* kbase;        // k_cache (layer applied) + the KV head's offset, bytes
  const char* vbase;
  const int32_t* table;     // the sequence's block-table row
  int64_t block_bytes;      // bytes between physical blocks
  int num_blocks;
  int block_shift;
  int bmask;
};

// One query row's running state, per lane: this lane group's share of the
// online softmax for the G query heads of the KV head.
template <bool BF16, int D, int G>
struct RowState {
  static constexpr int kVec = Vec16<BF16>::kN;
  float m[G], l[G], acc[G][kVec];
};

// Online softmax over the lane group's tokens of [start, end): token t =
// start + grp, start + grp + TPW, ...  `fresh_pos` (fused append) reads that
// position's K/V from the new-row buffers instead of the cache.  A table entry
// outside the pool sets `bad` and reads block 0 instead (the caller poisons).
template <bool BF16, int D, int G>
__device__ inline void row_walk(RowState<BF16, D, G>& st, const ValuView& c,
                                const float (&qf)[G][Vec16<BF16>::kN], int start, int end,
                                float scale_log2, int sub, int grp, int fresh_pos,
                                const char* fresh_k, const char* fresh_v, bool& bad) {
  using V = Vec16<BF16>;
  constexpr int kVec = V::kN;
  constexpr int kLpt = D / kVec;
  constexpr int kTpw = 64 / kLpt;
  constexpr int kElem = BF16 ? 2 : 4;
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.0f;
    for (int e = 0; e < kVec; ++e) st.acc[g][e] = 0.0f;
  }
  for (int t = start + grp; t < end; t += kTpw) {
    int phys = c.table[t >> c.block_shift];
    if (phys < 0 || phys >= c.num_blocks) {  // corrupt table entry: poison, never read it
      bad = true;
      phys = 0;
    }
    const int64_t byte_off =
        (int64_t)phys * c.block_bytes + ((int64_t)(t & c.bmask) * D + sub * kVec) * kElem;
    const bool fresh = t == fresh_pos;
    const char* kp = fresh ? fresh_k + sub * kVec * kElem : c.kbase + byte_off;
    const char* vp = fresh ? fresh_v + sub * kVec * kElem : c.vbase + byte_off;
    float kf[kVec], vf[kVec];
    V::unpack(*(const u32x4*)kp, kf);
    V::unpack(*(const u32x4*)vp, vf);
    for (int g = 0; g < G; ++g) {
      float dot = 0.0f;
      for (int e = 0; e < kVec; ++e) dot = fmaf(qf[g][e], kf[e], dot);
      for (int o = 1; o < kLpt; o <<= 1) dot += __shfl_xor(dot, o);
      const float sc = dot * scale_log2;
      const float mn = fmaxf(st.m[g], sc);
      const float keep = exp2f(st.m[g] - mn);  // 0 on the group's first token
      const float pe = exp2f(sc - mn);
      st.l[g] = st.l[g] * keep + pe;
      for (int e = 0; e < kVec; ++e) st.acc[g][e] = fmaf(pe, vf[e], st.acc[g][e] * keep);
      st.m[g] = mn;
    }
  }
}

// Merge the TPW lane groups' states: pairwise (m, l, acc) combination.  Every
// lane group ends with the whole row's state.
template <bool BF16, int D, int G>
__device__ inline void row_merge(RowState<BF16, D, G>& st) {
  constexpr int kVec = Vec16<BF16>::kN;
  constexpr int kLpt = D / kVec;
  for (int o = kLpt; o < 64; o <<= 1) {
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(st.m[g], o);
      const float lo = __shfl_xor(st.l[g], o);
      const float mn = fmaxf(st.m[g], mo);
      const float a = st.m[g] == -INFINITY ? 0.0f : exp2f(st.m[g] - mn);
      const float b = mo == -INFINITY ? 0.0f : exp2f(mo - mn);
      st.l[g] = st.l[g] * a + lo * b;
      for (int e = 0; e < kVec; ++e) {
        const float ao = __shfl_xor(st.acc[g][e], o);
        st.acc[g][e] = st.acc[g][e] * a + ao * b;
      }
      st.m[g] = mn;
    }
  }
}

// The query row's G heads (their slices of head_dim for this lane), as fp32.
template <bool BF16, int D, int G>
__device__ inline void load_q(float (&qf)[G][Vec16<BF16>::kN], const void* q, int64_t row0,
                              int sub) {
  constexpr int kVec = Vec16<BF16>::kN;
  constexpr int kElem = BF16 ? 2 : 4;
  for (int g = 0; g < G; ++g) {
    const u32x4 raw = *(const u32x4*)((const char*)q + ((row0 + g) * D + sub * kVec) * kElem);
    Vec16<BF16>::unpack(raw, qf[g]);
  }
}

template <bool BF16, int D, int G>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeParams p) {
  using V = Vec16<BF16>;
  constexpr int kVec = V::kN;        // values per lane per row
  constexpr int kLpt = D / kVec;     // lanes per token row
  constexpr int kElem = BF16 ? 2 : 4;
  static_assert(kLpt >= 1 && kLpt <= 64 && (64 % kLpt) == 0, "row must tile the wave");

  const WorkItem w = decode_work_item(p, blockIdx.x);
  const int lane = threadIdx.x;
  const int sub = lane % kLpt;       // which 16-byte slice of the row
  const int grp = lane / kLpt;       // which token stream
  const int len = p.seq_lens[w.seq];
  const int64_t out_row0 = (int64_t)w.seq * p.num_heads + (int64_t)w.head * G;
  // layered pool: layer blockIdx.y of the launch (0 for one per-layer pool)
  const int64_t layer = blockIdx.y;
  char* out = (char*)p.out + layer * p.layer_q_stride * kElem;
  const char* q = (const char*)p.q + layer * p.layer_q_stride * kElem;

  if (!seq_len_ok(p, len) || len == 0) {
    if (w.part == 0) store_new_token(p, w.seq, w.head, D * kElem, lane);
    if (w.part == 0 && grp == 0) {
      const float fill = len == 0 ? 0.0f : __builtin_nanf("");
      for (int g = 0; g < G; ++g)
        for (int e = 0; e < kVec; ++e) V::store(out, (out_row0 + g) * D + sub * kVec + e, fill);
    }
    return;
  }
  const int pstart = w.part * p.partition_size;
  if (pstart >= len) return;
  const int pend = range_end(pstart, p.partition_size, len);
  const int nparts = ceil_div_i(len, p.partition_size);

  float qf[G][kVec];
  load_q<BF16, D, G>(qf, q, out_row0, sub);

  const int64_t head_bytes = (int64_t)p.block_size * D * kElem;
  ValuView c;
  c.kbase = (const char*)p.k_cache + layer * p.layer_kv_stride * kElem + w.head * head_bytes;
  c.vbase = (const char*)p.v_cache + layer * p.layer_kv_stride * kElem + w.head * head_bytes;
  c.table = p.block_tables + (int64_t)w.seq * p.max_blocks_per_seq;
  c.block_bytes = p.block_stride != 0 ? p.block_stride * kElem : p.kv_heads * head_bytes;
  c.num_blocks = p.num_blocks;
  c.block_shift = p.block_shift;
  c.bmask = p.block_size - 1;

  const NewToken nt = new_token(p, w.seq, w.head, len, D * kElem);
  RowState<BF16, D, G> st;
  bool bad = false;
  row_walk<BF16, D, G>(st, c, qf, pstart, pend, p.scale_log2, sub, grp, nt.pos, nt.krow,
                       nt.vrow, bad);
  if (bad) {
    for (int g = 0; g < G; ++g) {
      st.l[g] = __builtin_nanf("");
      for (int e = 0; e < kVec; ++e) st.acc[g][e] = __builtin_nanf("");
    }
  }
  row_merge<BF16, D, G>(st);

  // fused append: the cache write comes after every cache read of this group
  if (w.part == 0) store_new_token(p, w.seq, w.head, D * kElem, lane);
  if (grp != 0) return;
  if (nparts == 1) {
    for (int g = 0; g < G; ++g) {
      const float inv = 1.0f / st.l[g];
      for (int e = 0; e < kVec; ++e)
        V::store(out, (out_row0 + g) * D + sub * kVec + e, st.acc[g][e] * inv);
    }
  } else {
    float* ws_o = p.ws_o + layer * p.layer_ws_stride;
    float* ws_ml = p.ws_ml + layer * (p.layer_ws_stride / D) * 2;
    for (int g = 0; g < G; ++g) {
      const int64_t slot = (out_row0 + g) * p.num_partitions + w.part;
      for (int e = 0; e < kVec; ++e) ws_o[slot * D + sub * kVec + e] = st.acc[g][e];
      if (sub == 0) {
        ws_ml[slot * 2 + 0] = st.m[g];
        ws_ml[slot * 2 + 1] = st.l[g];
      }
    }
  }
}

// Chunked prefill, one work-group per (sequence, KV head, tile of
// kPrefillValuRows chunk queries); grid index = (tile * num_seqs + seq) *
// kv_heads + head.  Same servability rules as the matrix-core prefill: a
// chunk longer than its sequence or than max_query_len, or a sequence longer
// than its table, gets NaN rows (written by tile 0); offsets out of range or
// decreasing skip the sequence.
template <bool BF16, int D, int G>
__global__ __launch_bounds__(64) void prefill_valu_kernel(PrefillParams p) {
  using V = Vec16<BF16>;
  constexpr int kVec = V::kN;
  constexpr int kLpt = D / kVec;
  constexpr int kElem = BF16 ? 2 : 4;
  const int head = blockIdx.x % p.kv_heads;
  const int rest = blockIdx.x / p.kv_heads;
  const int seq = rest % p.num_seqs;
  const int tile = rest / p.num_seqs;
  const int q0 = p.query_start[seq];
  const int q1 = p.query_start[seq + 1];
  if (q0 < 0 || q1 > p.num_queries || q1 <= q0) return;
  const int nq = q1 - q0;
  const int len = p.seq_lens[seq];
  const int lane = threadIdx.x;
  const int sub = lane % kLpt;
  const int grp = lane / kLpt;
  const bool servable = nq <= len && nq <= p.max_query_len &&
                        (int64_t)len <= (int64_t)p.max_blocks_per_seq * p.block_size;
  if (!servable) {
    if (tile != 0 || grp != 0) return;
    for (int i = 0; i < nq; ++i)
      for (int g = 0; g < G; ++g)
        for (int e = 0; e < kVec; ++e)
          V::store(p.out, ((int64_t)(q0 + i) * p.num_heads + (int64_t)head * G + g) * D +
                              sub * kVec + e,
                   __builtin_nanf(""));
    return;
  }
  const int i0 = tile * kPrefillValuRows;
  if (i0 >= nq) return;
  const int i1 = min(nq, i0 + kPrefillValuRows);
  const int pos0 = len - nq;  // position of chunk query 0

  const int64_t head_bytes = (int64_t)p.block_size * D * kElem;
  ValuView c;
  c.kbase = (const char*)p.k_cache + head * head_bytes;
  c.vbase = (const char*)p.v_cache + head * head_bytes;
  c.table = p.block_tables + (int64_t)seq * p.max_blocks_per_seq;
  c.block_bytes = p.kv_heads * head_bytes;
  c.num_blocks = p.num_blocks;
  c.block_shift = p.block_shift;
  c.bmask = p.block_size - 1;

  for (int i = i0; i < i1; ++i) {
    const int64_t row0 = (int64_t)(q0 + i) * p.num_heads + (int64_t)head * G;
    float qf[G][kVec];
    load_q<BF16, D, G>(qf, p.q, row0, sub);
    RowState<BF16, D, G> st;
    bool bad = false;
    row_walk<BF16, D, G>(st, c, qf, 0, pos0 + i + 1, p.scale_log2, sub, grp, -1, nullptr,
                         nullptr, bad);
    row_merge<BF16, D, G>(st);
    if (grp == 0) {
      for (int g = 0; g < G; ++g) {
        const float inv = bad ? __builtin_nanf("") : 1.0f / st.l[g];
        for (int e = 0; e < kVec; ++e)
          V::store(p.out, (row0 + g) * D + sub * kVec + e, st.acc[g][e] * inv);
      }
    }
  }
}

template <bool BF16, int D>
hipError_t launch_g(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.num_partitions * p.num_seqs * p.kv_heads),
                  (unsigned)(p.num_layers > 1 ? p.num_layers : 1));
  switch (p.group) {
    case 1: decode_valu_kernel<BF16, D, 1><<<grid, 64, 0, stream>>>(p); break;
    case 2: decode_valu_kernel<BF16, D, 2><<<grid, 64, 0, stream>>>(p); break;
    case 4: decode_valu_kernel<BF16, D, 4><<<grid, 64, 0, stream>>>(p); break;
    case 8: decode_valu_kernel<BF16, D, 8><<<grid, 64, 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_prefill_g(const PrefillParams& p, hipStream_t stream) {
  const int64_t tiles = ((int64_t)p.max_query_len + kPrefillValuRows - 1) / kPrefillValuRows;
  const int64_t wgs = tiles * p.num_seqs * p.kv_heads;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs);
  switch (p.group) {
    case 1: prefill_valu_kernel<BF16, D, 1><<<grid, 64, 0, stream>>>(p); break;
    case 2: prefill_valu_kernel<BF16, D, 2><<<grid, 64, 0, stream>>>(p); break;
    case 4: prefill_valu_kernel<BF16, D, 4><<<grid, 64, 0, stream>>>(p); break;
    case 8: prefill_valu_kernel<BF16, D, 8><<<grid, 64, 0, stream>>>(p); break;
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

hipError_t launch_prefill_valu(const PrefillParams& p, bool is_bf16, int head_dim,
                               hipStream_t stream) {
  if (is_bf16) {
    if (head_dim == 64) return launch_prefill_g<true, 64>(p, stream);
    if (head_dim == 128) return launch_prefill_g<true, 128>(p, stream);
  } else {
    if (head_dim == 64) return launch_prefill_g<false, 64>(p, stream);
    if (head_dim == 128) return launch_prefill_g<false, 128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
