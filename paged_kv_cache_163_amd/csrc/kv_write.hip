// KV append and copy-on-write block copy for gfx950.
//
// Both are byte moves: each thread moves one 16-byte vector (global_load_dwordx4 /
// global_store_dwordx4), consecutive threads take consecutive vectors of a row
// or block, so every wave reads and writes whole contiguous 1 KiB spans except
// at row ends.
#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// Append ("How PagedAttention works", section "A strong answer": each decode
// step adds one token's K and V to its sequence's cache).  Token i's row for KV head h goes to
// physical block slot/block_size, slot slot%block_size; blocks lie
// block_vecs 16-byte vectors apart (kv_heads * block_size * row_vecs for a
// per-layer pool, more in a layered pool where k_cache / v_cache point at
// one layer's K / V).
// Thread index -> (token, K or V, head, 16-byte vector of the row).
__global__ __launch_bounds__(kThreads) void kv_append_kernel(
    const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, const int64_t* __restrict__ slots, int num_tokens,
    int64_t num_slots, int kv_heads, int block_size, int row_vecs, int64_t block_vecs) {
  const int64_t per_token = 2ll * kv_heads * row_vecs;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)num_tokens * per_token) return;
  const int token = (int)(idx / per_token);
  int rem = (int)(idx - (int64_t)token * per_token);
  const int is_v = rem >= kv_heads * row_vecs;
  if (is_v) rem -= kv_heads * row_vecs;
  const int head = rem / row_vecs;
  const int vec = rem - head * row_vecs;
  const int64_t slot = slots[token];
  if (slot < 0 || slot >= num_slots) return;  // padding token / out of range: no write
  const int64_t block = slot / block_size;
  const int64_t offset = slot - block * block_size;
  const u32x4* src = (is_v ? v_new : k_new) + ((int64_t)token * kv_heads + head) * row_vecs + vec;
  u32x4* dst = (is_v ? v_cache : k_cache) + block * block_vecs +
               ((int64_t)head * block_size + offset) * row_vecs + vec;
  *dst = *src;
}

// Whole-block moves between two pools with the same block shape: the
// copy-on-write copy inside one pool ("How PagedAttention works", feature
// table: a fork copies only the block that diverges) and the preemption swap
// between the device pool and a pinned host pool (same table: swap blocks to
// host memory at block granularity).  Work-group index -> (pair, K or V,
// chunk of the block); the chunk loop strides by the grid's chunk count.
// Pairs naming a block outside either pool are skipped.  Host memory is
// reached through its device mapping, 16 bytes per lane.
// parts = 2: K and V pools (one block_vecs part of each per block, blocks
// block_vecs apart); parts = 1: one pool whose blocks (block_vecs each, K and
// V of every layer) are contiguous, the layered layout.
__global__ __launch_bounds__(kThreads) void move_blocks_kernel(
    u32x4* dst_k, u32x4* dst_v, int64_t dst_blocks, const u32x4* src_k, const u32x4* src_v,
    int64_t src_blocks, const int64_t* __restrict__ pairs, int64_t block_vecs, int chunks,
    int parts) {
  const int wg = blockIdx.x;
  const int chunk = wg % chunks;
  const int rest = wg / chunks;
  const int is_v = parts == 2 ? (rest & 1) : 0;
  const int pair = parts == 2 ? rest >> 1 : rest;
  const int64_t src = pairs[2 * pair];
  const int64_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const u32x4* from = (is_v ? src_v : src_k) + src * block_vecs;
  u32x4* to = (is_v ? dst_v : dst_k) + dst * block_vecs;
  for (int64_t i = (int64_t)chunk * kThreads + threadIdx.x; i < block_vecs;
       i += (int64_t)chunks * kThreads)
    to[i] = from[i];
}

}  // namespace

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int64_t* slots, int num_tokens, int64_t num_blocks,
                            int kv_heads, int block_size, int row_bytes, int64_t block_bytes,
                            hipStream_t stream) {
  const int row_vecs = row_bytes / 16;
  const int64_t total = (int64_t)num_tokens * 2 * kv_heads * row_vecs;
  const int64_t grid = (total + kThreads - 1) / kThreads;
  kv_append_kernel<<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
      (const u32x4*)k_new, (const u32x4*)v_new, (u32x4*)k_cache, (u32x4*)v_cache, slots,
      num_tokens, num_blocks * block_size, kv_heads, block_size, row_vecs, block_bytes / 16);
  return hipGetLastError();
}

hipError_t launch_move_blocks(void* dst_k, void* dst_v, int64_t dst_blocks, const void* src_k,
                              const void* src_v, int64_t src_blocks, const int64_t* pairs,
                              int num_pairs, int64_t block_bytes, hipStream_t stream) {
  const int parts = dst_v != nullptr ? 2 : 1;
  const int64_t block_vecs = block_bytes / 16;
  int64_t chunks = (block_vecs + kThreads - 1) / kThreads;
  if (chunks > 64) chunks = 64;  // each work-group then loops over its chunk stride
  const int64_t grid = (int64_t)num_pairs * parts * chunks;
  move_blocks_kernel<<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
      (u32x4*)dst_k, (u32x4*)dst_v, dst_blocks, (const u32x4*)src_k, (const u32x4*)src_v,
      src_blocks, pairs, block_vecs, (int)chunks, parts);
  return hipGetLastError();
}

}  // namespace pa
