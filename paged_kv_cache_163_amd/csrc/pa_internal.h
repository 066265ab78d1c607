// Internal declarations shared by the libpa.so translation units: the decode
// parameter block, small device helpers and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Shared-prefix decode: groups of consecutive sequences whose block tables
// start with the same physical blocks (one prefix, refcounted, many tables).
// Group g is sequences start[g] .. start[g+1] - 1; each of them shares the
// first tokens[g] / block_size table entries of sequence start[g] (its
// leader).  The prefix kernel attends every member's query over the shared
// keys once per group, in `parts` partitions of `partition` keys; the tail
// decode covers each member's positions [tokens[g], seq_len).  Carried in the
// kernel arguments (host arrays), so it costs no device memory.
constexpr int kMaxPrefixGroups = 32;
struct PrefixGroups {
  int32_t num_groups;           // 0: no sharing (every other decode launch)
  int32_t partition;            // prefix keys per prefix partition (a multiple of 32)
  int32_t parts;                // workspace slots of prefix partials per row (max over groups)
  int32_t start[kMaxPrefixGroups + 1];
  int32_t tokens[kMaxPrefixGroups];    // shared prefix tokens (whole blocks)
  int32_t wg_start[kMaxPrefixGroups + 1];  // prefix kernel: first work-group of each group
};

// Shared prefix tokens of sequence `seq` (0 outside every group).
__device__ inline int shared_prefix_tokens(const PrefixGroups& g, int seq) {
  int t = 0;
  for (int i = 0; i < g.num_groups; ++i)
    if (seq >= g.start[i] && seq < g.start[i + 1]) t = g.tokens[i];
  return t;
}

// Group of sequence `seq`, or -1.
__device__ inline int shared_prefix_group(const PrefixGroups& g, int seq) {
  int r = -1;
  for (int i = 0; i < g.num_groups; ++i)
    if (seq >= g.start[i] && seq < g.start[i + 1]) r = i;
  return r;
}

// Everything a decode launch needs, passed by value as the kernel argument.
struct DecodeParams {
  void* out;                    // [B][Hq][D] dtype
  const void* q;                // [B][Hq][D] dtype
  const void* k_cache;          // [NB][Hkv][BS][D] dtype
  const void* v_cache;
  const int32_t* block_tables;  // [B][max_blocks_per_seq]
  const int32_t* seq_lens;      // [B]
  float* ws_o;                  // [B][Hq][num_partitions][D]   unnormalised partial outputs
  float* ws_ml;                 // [B][Hq][num_partitions][2]   (running max, running sum)
  const void* k_new;            // fused append: [B][Hkv][D] new token per sequence, or null
  const void* v_new;
  const int64_t* new_slots;     // fused append: [B] cache slot of each new token (< 0: none)
  void* k_cache_w;              // fused append: writable views of the caches
  void* v_cache_w;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t kv_heads;
  int32_t group;                // num_heads / kv_heads
  int32_t max_blocks_per_seq;
  int32_t max_seq_len;
  int32_t num_blocks;
  int32_t block_size;           // power of two
  int32_t block_shift;          // log2(block_size)
  int32_t partition_size;       // tokens per partition
  int32_t num_partitions;       // grid extent along partitions
  int32_t waves;                // matrix-core kernel: waves per work-group (2 or 4)
  int32_t wave_parts;           // matrix-core kernel: 1 = each wave owns one partition
  float scale_log2;             // scale * log2(e): scores kept in base-2 units
  // Layered pool (decode over [NB][2][L][Hkv][BS][D]): k_cache / v_cache point
  // at the first decoded layer's K / V, blocks lie block_stride elements
  // apart, and launch layer y = blockIdx.y adds y * layer_kv_stride to both
  // caches, y * layer_q_stride to q and out and y * layer_ws_stride to ws_o
  // (y * layer_ws_stride / D * 2 to ws_ml).  Unused (0) for one per-layer pool.
  int64_t block_stride;
  int64_t layer_kv_stride;
  int64_t layer_q_stride;
  int64_t layer_ws_stride;
  int32_t num_layers;           // grid extent along layers (1 without layering)
  // Caller's processing order (a permutation of [0, num_seqs), longest
  // sequence first): work item slot s serves sequence order[s].  Null: the
  // kernel ranks the batch itself.
  const int32_t* order;
  // Shared-prefix decode (pa_decode_shared_prefix): the tail mode of the
  // matrix-core kernel starts each sequence after its shared prefix and
  // writes partials to slots prefix.parts + partition; the prefix kernel
  // writes slots [0, prefix.parts).  num_partitions counts both.
  PrefixGroups prefix;
};

// Everything a chunked-prefill launch needs.
struct PrefillParams {
  void* out;                    // [T][Hq][D] dtype
  const void* q;                // [T][Hq][D] dtype: sequence s's chunk is rows query_start[s]..
  const void* k_cache;          // [NB][Hkv][BS][D] dtype, the chunks already appended
  const void* v_cache;
  const int32_t* block_tables;  // [B][max_blocks_per_seq]
  const int32_t* seq_lens;      // [B] cached positions, chunk included
  const int32_t* query_start;   // [B+1] chunk offsets into q / out
  int32_t num_seqs;
  int32_t num_queries;          // T
  int32_t max_query_len;        // host bound on any chunk
  int32_t num_heads;
  int32_t kv_heads;
  int32_t group;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t block_size;
  int32_t block_shift;
  int32_t q_tiles;              // query tiles per (sequence, KV head)
  float scale_log2;
};

// Work-group index -> (kv head, sequence, partition).  Partition-major so that
// every sequence's first partition is dispatched before any second one, and
// consecutive work-groups (which the dispatcher spreads over the XCDs) walk
// the KV heads of one sequence.
struct WorkItem {
  int head;
  int seq;
  int part;
};

__device__ inline WorkItem decode_work_item(const DecodeParams& p, int wg) {
  WorkItem w;
  w.head = wg % p.kv_heads;
  const int rest = wg / p.kv_heads;
  w.seq = rest % p.num_seqs;
  w.part = rest / p.num_seqs;
  return w;
}

// ceil(a / b) for b > 0 without forming a + b - 1 (partition sizes may be
// close to INT32_MAX); 0 for a <= 0.
__device__ inline int ceil_div_i(int a, int b) { return a <= 0 ? 0 : (a - 1) / b + 1; }

// End of the range of at most `size` positions starting at `start`, cut at
// `limit` (start < limit), without forming start + size.
__device__ inline int range_end(int start, int size, int limit) {
  return limit - start <= size ? limit : start + size;
}

// A sequence length the grid and the table can serve.
__device__ inline bool seq_len_ok(const DecodeParams& p, int len) {
  return len >= 0 && len <= p.max_seq_len &&
         (int64_t)len <= ((int64_t)p.max_blocks_per_seq << p.block_shift);
}

// Fused append: the new token of sequence `seq` (position len - 1), if any:
// its cache slot and the row pointers of its KV head `head`; pos < 0 when
// there is none (the sequence's slot is negative).
struct NewToken {
  int pos;
  int64_t slot;
  const char* krow;
  const char* vrow;
};

__device__ inline NewToken new_token(const DecodeParams& p, int seq, int head, int len,
                                     int row_bytes) {
  NewToken t;
  t.slot = p.new_slots != nullptr ? p.new_slots[seq] : -1;
  // Wave-uniform by construction; readfirstlane keeps it (and every bound
  // derived from it) in scalar registers.
  t.pos = __builtin_amdgcn_readfirstlane(t.slot >= 0 && len > 0 ? len - 1 : -1);
  const int64_t off = ((int64_t)seq * p.kv_heads + head) * row_bytes;
  t.krow = (const char*)p.k_new + off;
  t.vrow = (const char*)p.v_new + off;
  return t;
}

// Fused append: thread `tid` < 2*row_bytes/16 of the caller holds 16 bytes of
// sequence `seq`'s new row for `head`: threads [0, row_bytes/16) the K row,
// the rest the V row.  Staged in LDS, the K row comes first and the V row
// follows it, so thread `tid`'s part goes to byte 16*tid.
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ inline nt_u32x4 new_row_part(const DecodeParams& p, int seq, int head, int row_bytes,
                                        int tid) {
  const int vecs = row_bytes / 16;
  const bool is_v = tid >= vecs;
  const int64_t src = ((int64_t)seq * p.kv_heads + head) * row_bytes + (is_v ? tid - vecs : tid) * 16;
  return *(const nt_u32x4*)((const char*)(is_v ? p.v_new : p.k_new) + src);
}

// Fused append, cache side: thread `tid`'s part `v` of the new row goes to
// cache slot `slot` of KV head `head`.  Negative slots and slots outside the
// pool are not written, as in pa_kv_append.  Kernels call this after their
// last cache read: a global store that may precede a load makes the compiler
// give up scalar loads for it (the block-table reads), because the scalar
// cache is not coherent with vector stores.
__device__ inline void store_row_part(const DecodeParams& p, int64_t slot, int head,
                                      int row_bytes, int tid, nt_u32x4 v) {
  const int vecs = row_bytes / 16;
  if (tid >= 2 * vecs || slot < 0 || slot >= (int64_t)p.num_blocks * p.block_size) return;
  const bool is_v = tid >= vecs;
  const int64_t block = slot >> p.block_shift;
  const int64_t off = slot & (p.block_size - 1);
  const int64_t dst = (((block * p.kv_heads + head) << p.block_shift) + off) * row_bytes +
                      (is_v ? tid - vecs : tid) * 16;
  *(nt_u32x4*)((char*)(is_v ? p.v_cache_w : p.k_cache_w) + dst) = v;
}

// The same, reading the slot and the row part itself.
__device__ inline void store_new_token(const DecodeParams& p, int seq, int head, int row_bytes,
                                       int tid) {
  if (p.new_slots == nullptr || tid >= 2 * (row_bytes / 16)) return;
  store_row_part(p, p.new_slots[seq], head, row_bytes, tid,
                 new_row_part(p, seq, head, row_bytes, tid));
}

// bfloat16 <-> fp32.  A bf16 is the top half of a binary32.
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);  // v_cvt_pk_bf16_f32: nearest-even
}

// ---- launchers (return the launch status) --------------------------------
hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int64_t* slots, int num_tokens, int64_t num_blocks,
                            int kv_heads, int block_size, int row_bytes, int64_t block_bytes,
                            hipStream_t stream);

// dst_v == nullptr: one-part pools (the layered layout, whole blocks of
// block_bytes); otherwise K and V pools with block_bytes per part.
hipError_t launch_move_blocks(void* dst_k, void* dst_v, int64_t dst_blocks, const void* src_k,
                              const void* src_v, int64_t src_blocks, const int64_t* pairs,
                              int num_pairs, int64_t block_bytes, hipStream_t stream);

// is_bf16: element type of q/out/caches; head_dim in {64, 128}; group in {1,2,4,8}.
// Rows of (position, query head) one prefill work-group covers.
constexpr int kPrefillRows = 128;
hipError_t launch_prefill_mfma(const PrefillParams& p, int head_dim, hipStream_t stream);

// Vector-ALU decode: fp32 or bf16, head_dim in {64, 128}, group in {1,2,4,8},
// any power-of-two block size; per-layer or layered pools (grid y = layers).
hipError_t launch_decode_valu(const DecodeParams& p, bool is_bf16, int head_dim,
                              hipStream_t stream);

// Vector-ALU chunked prefill for the shapes the matrix-core prefill does not
// take (fp32, block sizes below 16): same arguments and results.  A
// work-group covers kPrefillValuRows chunk queries of one (sequence, KV head).
constexpr int kPrefillValuRows = 8;
hipError_t launch_prefill_valu(const PrefillParams& p, bool is_bf16, int head_dim,
                               hipStream_t stream);

// bf16 only; head_dim in {64, 128}; block_size >= 16; group <= 16;
// partition_size a multiple of 32.
hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, hipStream_t stream);

// Merges the per-partition partials of sequences with more than one partition.
hipError_t launch_decode_reduce(const DecodeParams& p, bool is_bf16, int head_dim,
                                hipStream_t stream);

// Shared-prefix decode, bf16, head_dim in {64, 128}, group a power of two
// <= 16, block_size >= 16: one launch of the prefix attention (every group
// member's query over the group's shared keys; p.prefix.wg_start[num_groups]
// work-groups) and the tail decode (num_partitions - prefix.parts partitions
// per sequence and KV head), partials to the workspace.
hipError_t launch_shared_prefix(const DecodeParams& p, int head_dim, hipStream_t stream);
// Merge of prefix and tail partials, one work-group per (sequence, KV head);
// also checks that members' tables start with their leader's blocks.
hipError_t launch_prefix_merge(const DecodeParams& p, int head_dim, hipStream_t stream);

}  // namespace pa
