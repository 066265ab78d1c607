// Host-side block bookkeeping of the paged KV cache (include/pa.h, pa_bm_*):
// the steps either side of pa_kv_append / pa_copy_blocks / pa_swap_blocks.
//
// "How PagedAttention works", section "A strong answer": the pool is split
// into blocks of one size, every sequence has its own table of block ids and
// at most its final block has unused slots; the feature table: a shared
// prefix is a single set of blocks counted by reference, a fork shares its
// parent's blocks and copies a block only when one branch writes to it,
// preemption moves whole blocks out to host memory.  Section "What
// interviewers probe next": a request is admitted when the pool has
// ceil(prompt / block size) blocks for it plus one to grow into, above a
// small watermark reserve.
//
// Policies the pages leave open: the lowest-numbered free block is taken
// first (so placements are reproducible); the watermark gates admission only;
// a batch of appends is all or nothing; swap-out copies each of a sequence's
// blocks to its own host block (blocks shared with resident sequences stay on
// the device for them) and swap-in gives each host block a fresh device
// block.  A swapped-out sequence cannot grow, fork or be decoded.
//
// Plain host C++: no HIP calls.  A manager is not thread-safe; callers
// serialise access to one manager.
#include <stdint.h>

#include <algorithm>
#include <functional>
#include <new>
#include <queue>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pa.h"

namespace {

// One pool (device or pinned host): reference counts and a min-heap of free ids.
class Pool {
 public:
  explicit Pool(int64_t n) : ref_(n, 0) {
    std::vector<int32_t> ids(n);
    for (int64_t i = 0; i < n; ++i) ids[i] = (int32_t)i;
    free_ = Heap(std::greater<int32_t>(), std::move(ids));
  }
  int64_t size() const { return (int64_t)ref_.size(); }
  int64_t num_free() const { return (int64_t)free_.size(); }
  int32_t ref(int64_t b) const { return ref_[b]; }
  int32_t take() {
    const int32_t b = free_.top();
    free_.pop();
    ref_[b] = 1;
    return b;
  }
  void share(int32_t b) { ++ref_[b]; }
  void drop(int32_t b) {
    if (--ref_[b] == 0) free_.push(b);
  }

 private:
  using Heap = std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>>;
  std::vector<int32_t> ref_;
  Heap free_;
};

struct Seq {
  std::vector<int32_t> blocks;  // device ids, or host ids while swapped out
  int64_t len = 0;              // cached positions
  bool swapped = false;
};

int64_t blocks_for(int64_t tokens, int64_t b) { return (tokens + b - 1) / b; }

}  // namespace

struct pa_block_manager {
  pa_block_manager(int64_t nb, int32_t bs, int64_t wm, int64_t nh)
      : block_size(bs), watermark(wm), dev(nb), host(nh) {}
  int32_t block_size;
  int64_t watermark;
  Pool dev;
  Pool host;
  std::unordered_map<int64_t, Seq> seqs;

  Seq* resident(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() || it->second.swapped ? nullptr : &it->second;
  }
  bool needs_block(const Seq& s) const {
    return s.len % block_size == 0 || dev.ref(s.blocks.back()) > 1;
  }
};

extern "C" {

pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, int64_t watermark_blocks,
                       int64_t num_host_blocks, pa_block_manager** out) {
  if (!out || num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0 ||
      watermark_blocks < 0 || num_host_blocks < 0 || num_host_blocks > INT32_MAX)
    return PA_ERR_INVALID_ARG;
  *out = new (std::nothrow) pa_block_manager(num_blocks, block_size, watermark_blocks,
                                             num_host_blocks);
  return *out ? PA_OK : PA_ERR_NO_SPACE;
}

pa_status pa_bm_destroy(pa_block_manager* bm) {
  delete bm;
  return PA_OK;
}

pa_status pa_bm_can_admit(const pa_block_manager* bm, int64_t prompt_tokens, int32_t* ok) {
  if (!bm || !ok || prompt_tokens < 0) return PA_ERR_INVALID_ARG;
  const int64_t need = blocks_for(prompt_tokens, bm->block_size) + 1;
  *ok = bm->dev.num_free() - bm->watermark >= need;
  return PA_OK;
}

pa_status pa_bm_admit(pa_block_manager* bm, int64_t seq, int64_t prompt_tokens) {
  int32_t ok = 0;
  const pa_status st = pa_bm_can_admit(bm, prompt_tokens, &ok);
  if (st != PA_OK) return st;
  if (bm->seqs.count(seq)) return PA_ERR_INVALID_ARG;
  if (!ok) return PA_ERR_NO_SPACE;
  Seq s;
  s.len = prompt_tokens;
  const int64_t n = blocks_for(prompt_tokens, bm->block_size);
  s.blocks.reserve(n + 1);
  for (int64_t i = 0; i < n; ++i) s.blocks.push_back(bm->dev.take());
  bm->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return PA_ERR_INVALID_ARG;
  Seq* p = bm->resident(parent);
  if (!p || bm->seqs.count(child)) return PA_ERR_INVALID_ARG;
  Seq c;
  c.blocks = p->blocks;
  c.len = p->len;
  for (int32_t b : c.blocks) bm->dev.share(b);
  bm->seqs.emplace(child, std::move(c));
  return PA_OK;
}

pa_status pa_bm_append_slots(pa_block_manager* bm, const int64_t* seqs, int32_t n,
                             int64_t* slots, int64_t* cow_pairs, int32_t* num_cow) {
  if (!bm || n < 0 || (n > 0 && (!seqs || !slots || !cow_pairs)) || !num_cow)
    return PA_ERR_INVALID_ARG;
  std::vector<Seq*> batch(n);
  std::unordered_set<int64_t> seen;
  int64_t fresh = 0;
  for (int32_t i = 0; i < n; ++i) {
    batch[i] = bm->resident(seqs[i]);
    if (!batch[i] || !seen.insert(seqs[i]).second) return PA_ERR_INVALID_ARG;
    fresh += bm->needs_block(*batch[i]);
  }
  if (fresh > bm->dev.num_free()) return PA_ERR_NO_SPACE;  // nothing changed
  const int64_t b = bm->block_size;
  int32_t ncow = 0;
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = *batch[i];
    const int64_t pos = s.len;
    if (pos % b == 0) {
      s.blocks.push_back(bm->dev.take());
    } else if (bm->dev.ref(s.blocks.back()) > 1) {
      const int32_t shared = s.blocks.back();
      const int32_t copy = bm->dev.take();
      bm->dev.drop(shared);
      s.blocks.back() = copy;
      cow_pairs[2 * ncow] = shared;
      cow_pairs[2 * ncow + 1] = copy;
      ++ncow;
    }
    slots[i] = (int64_t)s.blocks[pos / b] * b + pos % b;
    s.len = pos + 1;
  }
  *num_cow = ncow;
  return PA_OK;
}

pa_status pa_bm_release(pa_block_manager* bm, int64_t seq) {
  if (!bm) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
  Pool& pool = it->second.swapped ? bm->host : bm->dev;
  for (int32_t b : it->second.blocks) pool.drop(b);
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_swap_out(pa_block_manager* bm, int64_t seq, int64_t* pairs, int64_t capacity,
                         int64_t* num_pairs) {
  if (!bm || !num_pairs) return PA_ERR_INVALID_ARG;
  Seq* s = bm->resident(seq);
  if (!s) return PA_ERR_INVALID_ARG;
  const int64_t n = (int64_t)s->blocks.size();
  if (capacity < n || (n > 0 && !pairs)) return PA_ERR_INVALID_ARG;
  if (n > bm->host.num_free()) return PA_ERR_NO_SPACE;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t h = bm->host.take();
    pairs[2 * i] = s->blocks[i];
    pairs[2 * i + 1] = h;
    bm->dev.drop(s->blocks[i]);
    s->blocks[i] = h;
  }
  s->swapped = true;
  *num_pairs = n;
  return PA_OK;
}

pa_status pa_bm_swap_in(pa_block_manager* bm, int64_t seq, int64_t* pairs, int64_t capacity,
                        int64_t* num_pairs) {
  if (!bm || !num_pairs) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end() || !it->second.swapped) return PA_ERR_INVALID_ARG;
  Seq& s = it->second;
  const int64_t n = (int64_t)s.blocks.size();
  if (capacity < n || (n > 0 && !pairs)) return PA_ERR_INVALID_ARG;
  if (n > bm->dev.num_free()) return PA_ERR_NO_SPACE;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t d = bm->dev.take();
    pairs[2 * i] = s.blocks[i];
    pairs[2 * i + 1] = d;
    bm->host.drop(s.blocks[i]);
    s.blocks[i] = d;
  }
  s.swapped = false;
  *num_pairs = n;
  return PA_OK;
}

pa_status pa_bm_decode_inputs(const pa_block_manager* bm, const int64_t* seqs, int32_t n,
                              int32_t max_blocks, int32_t pad_block, int32_t* tables,
                              int32_t* seq_lens) {
  if (!bm || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !tables || !seq_lens)))
    return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {  // validate the whole batch before writing
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end() || it->second.swapped ||
        (int64_t)it->second.blocks.size() > max_blocks || it->second.len > INT32_MAX)
      return PA_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = tables + (int64_t)i * max_blocks;
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    std::fill(row + s.blocks.size(), row + max_blocks, pad_block);
    seq_lens[i] = (int32_t)s.len;
  }
  return PA_OK;
}

pa_status pa_bm_sequence(const pa_block_manager* bm, int64_t seq, int64_t* len,
                         int64_t* num_blocks, int32_t* swapped) {
  if (!bm || !len || !num_blocks || !swapped) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
  *len = it->second.len;
  *num_blocks = (int64_t)it->second.blocks.size();
  *swapped = it->second.swapped;
  return PA_OK;
}

pa_status pa_bm_stats(const pa_block_manager* bm, int64_t* free_blocks, int64_t* free_host_blocks,
                      int64_t* num_seqs) {
  if (!bm || !free_blocks || !free_host_blocks || !num_seqs) return PA_ERR_INVALID_ARG;
  *free_blocks = bm->dev.num_free();
  *free_host_blocks = bm->host.num_free();
  *num_seqs = (int64_t)bm->seqs.size();
  return PA_OK;
}

pa_status pa_bm_refcount(const pa_block_manager* bm, int64_t block, int32_t host, int32_t* ref) {
  if (!bm || !ref) return PA_ERR_INVALID_ARG;
  const Pool& pool = host ? bm->host : bm->dev;
  if (block < 0 || block >= pool.size()) return PA_ERR_INVALID_ARG;
  *ref = pool.ref(block);
  return PA_OK;
}

}  // extern "C"
