// C ABI of libpa.so (declared in include/pa.h): argument checks, decode
// planning (kernel, partition size, grid, workspace) and kernel dispatch.
// Every check on host-side arguments runs before anything is launched; the
// only HIP calls before a launch are the device and compute-unit queries of
// the shared-prefix plan and the pointer-attribute queries of the block swap.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

constexpr int32_t kAbiVersion = 2;
// Work-groups a decode launch should offer before sequences are split: the
// two resident four-wave work-groups per compute unit of a 256-CU MI355X.
// Measured on 16 sequences x 8,192 tokens x 8 KV heads: 89 us at 2,048-token
// partitions (512 work-groups) against 91 us at 1,024 (1,024 work-groups,
// more partials to merge) and 129 us unsplit (128 work-groups).
constexpr int64_t kTargetWorkgroups = 512;
// ...but a split never makes partitions shorter than this: a short partition
// is mostly the fixed latency of its work-group, and the split adds the
// merge launch.  Measured on 256 sequences of 500-950 tokens with one KV
// head: 23.3 us unsplit (256 work-groups) against 27.6 us for two
// partitions of 480 tokens and 28.3 us for four of 256.
constexpr int64_t kMinSplitTokens = 1024;
constexpr int32_t kMfmaStep = 32;  // tokens per MFMA-kernel step
constexpr int64_t kMaxPartitions = 16384;  // partitions per sequence (split kernels)
constexpr int32_t kDefaultCus = 256;     // MI355X, used when no device is visible
constexpr int kMaxDevices = 64;

// Compute units of the current device (cached per device).
int32_t device_cus() {
  static std::atomic<int32_t> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kDefaultCus;
  }
  int32_t v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    return kDefaultCus;
  }
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Device scratch of pa_decode_noalloc: the split kernels' partials live here
// instead of in a caller workspace.  One copy per device, alive until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device array: kernels and copies get the address hipGetSymbolAddress
// returns for the current device (scratch_ptr).
constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on the current device, looked up once per device
// with that device current; nullptr when the lookup fails.
void* scratch_ptr() {
  static std::atomic<void*> ptrs[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* v = ptrs[dev].load(std::memory_order_acquire);
  if (v != nullptr) return v;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  ptrs[dev].store(addr, std::memory_order_release);
  return addr;
}

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr % a) == 0; }
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int32_t log2i(int64_t v) {
  int32_t s = 0;
  while ((int64_t(1) << s) < v) ++s;
  return s;
}
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
int32_t elem_bytes(int32_t dtype) { return dtype == PA_BF16 ? 2 : 4; }
bool dtype_ok(int32_t dtype) { return dtype == PA_F32 || dtype == PA_BF16; }

struct Plan {
  int32_t kernel;      // PA_KERNEL_VALU or PA_KERNEL_MFMA
  int32_t partition;   // tokens per partition
  int32_t partitions;  // grid extent along partitions
  int32_t waves;       // matrix-core kernel: waves per work-group
  int32_t wave_parts;  // matrix-core kernel: 1 = a partition per wave
  size_t workspace;    // bytes
};

// Work-group shape of the matrix-core decode.  Whole sequences (one
// partition each) vary in length, and four-wave work-groups, each wave taking
// every fourth 32-token step, dispatched longest first, keep the compute
// units evenly loaded to the end of the launch.  Equal partitions of a split
// need no such balance; what costs there is the fixed work per wave (the
// prologue, the cross-wave merge, the partial store), so each wave should
// walk many steps.  The GPU holds 8 waves per compute unit at this kernel's
// register use (two per SIMD).  A split with at least that many work items
// gives each wave of a four-wave work-group a partition of its own ("wave
// per partition": no cross-wave merge); one with half as many takes two-wave
// work-groups.  Measured on 16 sequences x 8,192 tokens x 8 KV heads (decode
// + reduce, one box): 512-token partitions (2,048 items) 94.6 us with a
// partition per wave, against 101.6-102.3 us with two or four waves sharing
// each partition (95.6 us with single-wave work-groups); 1,024-token
// partitions 89.8 us with two-wave work-groups against 91.0 with four;
// 2,048-token partitions (512 items) 88.4 us with four.
constexpr int32_t kWaveSlotsPerCu = 8;
struct WgShape {
  int32_t waves;
  int32_t wave_parts;
};
WgShape decode_shape(int64_t parts, int64_t grid) {
  if (parts <= 1) return {4, 0};
  const int64_t slots = (int64_t)kWaveSlotsPerCu * device_cus();
  if (grid >= slots) return {4, 1};
  if (grid >= slots / 2) return {2, 0};
  return {4, 0};
}

bool valu_supports(int32_t dtype, int32_t head_dim, int32_t group, int32_t block_size) {
  (void)dtype;
  return (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8) && pow2(block_size) &&
         block_size <= 256;
}

bool mfma_supports(int32_t dtype, int32_t head_dim, int32_t group, int32_t block_size) {
  return dtype == PA_BF16 && (head_dim == 64 || head_dim == 128) && group >= 1 && group <= 16 &&
         pow2(block_size) && block_size >= 16 && block_size <= 256;
}

pa_status make_plan(int32_t num_seqs, int32_t num_heads, int32_t kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_seq_len, int32_t partition_size,
                    int32_t dtype, int32_t kernel, Plan* plan) {
  if (num_seqs < 0 || num_heads <= 0 || kv_heads <= 0 || num_heads % kv_heads != 0 ||
      head_dim <= 0 || block_size <= 0 || max_seq_len < 0 || partition_size < 0 ||
      !dtype_ok(dtype))
    return PA_ERR_INVALID_ARG;
  if (kernel != PA_KERNEL_AUTO && kernel != PA_KERNEL_VALU && kernel != PA_KERNEL_MFMA)
    return PA_ERR_INVALID_ARG;
  if (!pow2(block_size) || block_size > 256) return PA_ERR_UNSUPPORTED;
  const int32_t group = num_heads / kv_heads;
  const bool mfma = mfma_supports(dtype, head_dim, group, block_size);
  const bool valu = valu_supports(dtype, head_dim, group, block_size);
  int32_t chosen;
  if (kernel == PA_KERNEL_MFMA) {
    if (!mfma) return PA_ERR_UNSUPPORTED;
    chosen = kernel;
  } else if (kernel == PA_KERNEL_VALU) {
    if (!valu) return PA_ERR_UNSUPPORTED;
    chosen = PA_KERNEL_VALU;
  } else {
    if (!mfma && !valu) return PA_ERR_UNSUPPORTED;
    chosen = mfma ? PA_KERNEL_MFMA : PA_KERNEL_VALU;
  }
  const int64_t granule = chosen == PA_KERNEL_MFMA ? kMfmaStep : 1;
  // A partition never needs to be longer than the longest sequence, so a
  // requested size is capped there (a huge request such as INT32_MAX means
  // "do not split"); every later sum of a start and a partition size then
  // stays within int32 on the device.
  const int64_t whole = round_up(max_seq_len > 0 ? max_seq_len : 1, granule);
  int64_t part;
  if (partition_size > 0) {
    part = round_up(partition_size, granule);
  } else {
    // Split only as far as needed to offer kTargetWorkgroups work-groups,
    // and only while every partition keeps kMinSplitTokens tokens.
    const int64_t units = (int64_t)num_seqs * kv_heads;
    int64_t splits = units >= kTargetWorkgroups || units == 0
                         ? 1
                         : ceil_div(kTargetWorkgroups, units);
    const int64_t longest = max_seq_len > 0 ? max_seq_len : 1;
    if (splits > longest / kMinSplitTokens) splits = longest / kMinSplitTokens;
    if (splits < 1) splits = 1;
    part = ceil_div(max_seq_len > 0 ? max_seq_len : 1, splits);
    if (part < 256) part = 256;
    part = round_up(part, chosen == PA_KERNEL_MFMA ? kMfmaStep : 16);
  }
  if (part > whole) part = whole;
  if (part > INT32_MAX - kMfmaStep) return PA_ERR_INVALID_ARG;
  const int64_t parts = max_seq_len > 0 ? ceil_div(max_seq_len, part) : 1;
  if (parts > kMaxPartitions) return PA_ERR_UNSUPPORTED;  // reduce kernel's LDS weights
  const int64_t grid = parts * (int64_t)num_seqs * kv_heads;
  if (grid > INT32_MAX) return PA_ERR_INVALID_ARG;
  plan->kernel = chosen;
  plan->partition = (int32_t)part;
  plan->partitions = (int32_t)parts;
  const WgShape shape = chosen == PA_KERNEL_MFMA ? decode_shape(parts, grid) : WgShape{1, 0};
  plan->waves = shape.waves;
  plan->wave_parts = shape.wave_parts;
  plan->workspace = parts > 1 ? (size_t)num_seqs * num_heads * parts * (head_dim + 2) * 4 : 0;
  return PA_OK;
}

pa_status from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// Where a pointer's memory lives, and the address a kernel uses for it.
enum Residency { kUnknown, kDevice, kPinnedHost };
Residency residency(const void* ptr, const void** kernel_ptr) {
  hipPointerAttribute_t a;
  if (ptr == nullptr || hipPointerGetAttributes(&a, ptr) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of a failed query
    return kUnknown;
  }
  if (a.type == hipMemoryTypeDevice) {
    *kernel_ptr = ptr;
    return kDevice;
  }
  if (a.type == hipMemoryTypeHost && a.devicePointer != nullptr && a.hostPointer != nullptr) {
    // the mapping must also be what the runtime hands out for this address
    const void* mapped =
        (const char*)a.devicePointer + ((const char*)ptr - (const char*)a.hostPointer);
    void* check = nullptr;
    if (hipHostGetDevicePointer(&check, const_cast<void*>(ptr), 0) != hipSuccess ||
        check != mapped) {
      (void)hipGetLastError();
      return kUnknown;
    }
    *kernel_ptr = mapped;
    return kPinnedHost;
  }
  return kUnknown;  // pageable host memory or a type a kernel cannot address
}

// Shared-prefix decode plan: the tail decode's plan on the matrix-core kernel
// (partitions over the positions after the prefix) plus the prefix
// partitions.  The prefix keys are split until the prefix work-groups fill
// about one of the two work-group slots of every compute unit
// (kPrefixWgsPerCu): they are dispatched first and run longest, and the tail
// work-groups stream through the other slot meanwhile.  prefix_partition_size
// > 0 fixes the split instead.  Groups with no member or no shared block
// share nothing.
constexpr int32_t kPrefixWgsPerCu = 1;
static_assert(pa::kMaxPrefixGroups == PA_MAX_PREFIX_GROUPS, "group limit");

pa_status shared_prefix_plan(int32_t num_seqs, int32_t num_heads, int32_t kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                             int32_t max_blocks_per_seq, const int32_t* group_start,
                             const int32_t* group_prefix_blocks, int32_t num_groups,
                             int32_t prefix_partition_size, int32_t partition_size, int32_t dtype,
                             Plan* plan, pa::PrefixGroups* pg) {
  Plan tail;
  const pa_status st = make_plan(num_seqs, num_heads, kv_heads, head_dim, block_size,
                                 max_seq_len, partition_size, dtype, PA_KERNEL_MFMA, &tail);
  if (st != PA_OK) return st;
  if (num_groups < 0 || prefix_partition_size < 0 || max_blocks_per_seq <= 0)
    return PA_ERR_INVALID_ARG;
  if (num_groups > pa::kMaxPrefixGroups) return PA_ERR_UNSUPPORTED;
  const int32_t group = num_heads / kv_heads;
  if (!pow2(group) || group > 16) return PA_ERR_UNSUPPORTED;  // 128 / group members per tile
  memset(pg, 0, sizeof(*pg));
  if (num_groups > 0) {
    if (group_start == nullptr || group_prefix_blocks == nullptr) return PA_ERR_INVALID_ARG;
    if (group_start[0] < 0) return PA_ERR_INVALID_ARG;
    for (int32_t g = 0; g < num_groups; ++g) {
      const int64_t blocks = group_prefix_blocks[g];
      if (group_start[g + 1] < group_start[g] || group_start[g + 1] > num_seqs || blocks < 0 ||
          blocks > max_blocks_per_seq || blocks * block_size > max_seq_len)
        return PA_ERR_INVALID_ARG;
    }
  }
  // work-groups of the prefix kernel without splitting the keys
  int64_t base = 0, max_tokens = 0;
  for (int32_t g = 0; g < num_groups; ++g) {
    const int64_t members = group_start[g + 1] - group_start[g];
    const int64_t tokens = (int64_t)group_prefix_blocks[g] * block_size;
    if (members == 0 || tokens == 0) continue;
    base += ceil_div(members * group, pa::kPrefillRows) * kv_heads;
    if (tokens > max_tokens) max_tokens = tokens;
  }
  *plan = tail;
  if (max_tokens == 0) return PA_OK;  // nothing shared: the plain decode
  int64_t part;
  if (prefix_partition_size > 0) {
    part = round_up(prefix_partition_size, kMfmaStep);
  } else {
    const int64_t target = (int64_t)kPrefixWgsPerCu * device_cus();
    const int64_t splits = base >= target ? 1 : target / base;
    part = round_up(ceil_div(max_tokens, splits), kMfmaStep);
  }
  // no prefix partition is longer than the longest prefix (a huge request
  // means "do not split"), which keeps the device's int32 sums in range
  const int64_t whole = round_up(max_tokens, kMfmaStep);
  if (part > whole) part = whole;
  if (part > INT32_MAX - kMfmaStep) return PA_ERR_INVALID_ARG;
  const int64_t parts = ceil_div(max_tokens, part);
  const int64_t slots = parts + tail.partitions;
  if (slots > kMaxPartitions || (int64_t)group * slots * 4 > 64 * 1024) return PA_ERR_UNSUPPORTED;
  pg->num_groups = num_groups;
  pg->partition = (int32_t)part;
  pg->parts = (int32_t)parts;
  int64_t wgs = 0;
  for (int32_t g = 0; g < num_groups; ++g) {
    const int64_t members = group_start[g + 1] - group_start[g];
    const int64_t tokens = (int64_t)group_prefix_blocks[g] * block_size;
    pg->start[g] = group_start[g];
    pg->tokens[g] = members > 0 ? (int32_t)tokens : 0;
    pg->wg_start[g] = (int32_t)wgs;
    if (members > 0 && tokens > 0)
      wgs += round_up(kv_heads * ceil_div(tokens, part), 8) *
             ceil_div(members * group, pa::kPrefillRows);
    if (wgs > INT32_MAX) return PA_ERR_INVALID_ARG;
  }
  pg->start[num_groups] = group_start[num_groups];
  pg->wg_start[num_groups] = (int32_t)wgs;
  plan->partitions = (int32_t)slots;
  plan->workspace = (size_t)num_seqs * num_heads * slots * (head_dim + 2) * 4;
  return PA_OK;
}

}  // namespace

// Decode over layers of a layered pool: k_cache / v_cache point at the first
// decoded layer, `layers` layers are decoded by one launch.
struct LayerSpec {
  int64_t block_stride;     // elements between physical blocks
  int64_t layer_kv_stride;  // elements between consecutive layers' K (and V)
  int32_t layers;
};

static pa_status decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* seq_lens, int32_t max_seq_len, int32_t num_seqs,
                             int32_t num_heads, int32_t kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks, float scale,
                             int32_t partition_size, void* workspace, size_t workspace_bytes,
                             int32_t dtype, int32_t kernel, void* stream, const void* k_new,
                             const void* v_new, const int64_t* new_slots,
                             const LayerSpec* lay = nullptr, const int32_t* order = nullptr) {
  Plan plan;
  const pa_status st = make_plan(num_seqs, num_heads, kv_heads, head_dim, block_size,
                                 max_seq_len, partition_size, dtype, kernel, &plan);
  if (st != PA_OK) return st;
  if (lay != nullptr) plan.workspace *= (size_t)lay->layers;  // a partial set per layer
  if (num_blocks <= 0 || max_blocks_per_seq <= 0 || !isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens) return PA_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4))
    return PA_ERR_INVALID_ARG;
  if (plan.workspace > 0 &&
      (workspace == nullptr || workspace_bytes < plan.workspace || !aligned(workspace, 16)))
    return PA_ERR_INVALID_ARG;
  const bool fused = new_slots != nullptr;
  if (fused) {
    if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(new_slots, 8))
      return PA_ERR_INVALID_ARG;
  }

  pa::DecodeParams p;
  memset(&p, 0, sizeof(p));
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  if (fused) {
    p.k_new = k_new;
    p.v_new = v_new;
    p.new_slots = new_slots;
    p.k_cache_w = (void*)k_cache;
    p.v_cache_w = (void*)v_cache;
  }
  if (plan.workspace > 0) {
    const size_t per_layer_o = (size_t)num_seqs * num_heads * plan.partitions * head_dim;
    p.ws_o = (float*)workspace;
    p.ws_ml = p.ws_o + per_layer_o * (lay != nullptr ? lay->layers : 1);
  }
  if (order != nullptr) {
    if (!aligned(order, 4)) return PA_ERR_INVALID_ARG;
    if (plan.kernel == PA_KERNEL_MFMA) p.order = order;  // the vector-ALU kernel ranks nothing
  }
  if (lay != nullptr) {
    p.block_stride = lay->block_stride;
    p.layer_kv_stride = lay->layer_kv_stride;
    p.layer_q_stride = (int64_t)num_seqs * num_heads * head_dim;
    p.layer_ws_stride = (int64_t)num_seqs * num_heads * plan.partitions * head_dim;
    p.num_layers = lay->layers;
  }
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.kv_heads = kv_heads;
  p.group = num_heads / kv_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_seq_len = max_seq_len;
  p.num_blocks = num_blocks;
  p.block_size = block_size;
  p.block_shift = log2i(block_size);
  p.partition_size = plan.partition;
  p.num_partitions = plan.partitions;
  // the fused append keeps one partition per work-group
  p.waves = fused && plan.wave_parts ? 4 : plan.waves;
  p.wave_parts = fused ? 0 : plan.wave_parts;
  p.scale_log2 = scale * 1.4426950408889634f;  // log2(e)

  const hipStream_t s = (hipStream_t)stream;
  const bool bf16 = dtype == PA_BF16;
  hipError_t e = plan.kernel == PA_KERNEL_MFMA ? pa::launch_decode_mfma(p, head_dim, s)
                                               : pa::launch_decode_valu(p, bf16, head_dim, s);
  if (e != hipSuccess) return PA_ERR_HIP;
  if (plan.partitions > 1) {
    e = pa::launch_decode_reduce(p, bf16, head_dim, s);
    if (e != hipSuccess) return PA_ERR_HIP;
  }
  return PA_OK;
}


extern "C" {

int32_t pa_abi_version(void) { return kAbiVersion; }

const char* pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PA_ERR_HIP: return "HIP launch error";
    case PA_ERR_NO_SPACE: return "not enough free blocks";
    case PA_ERR_SCRATCH: return "workspace need exceeds the library's static scratch";
    default: return "unknown status";
  }
}

pa_status pa_block_layout(int64_t tokens, int32_t block_size, int64_t* blocks, int64_t* unused) {
  if (tokens < 0 || block_size <= 0 || blocks == nullptr || unused == nullptr)
    return PA_ERR_INVALID_ARG;
  const int64_t n = tokens / block_size + (tokens % block_size != 0 ? 1 : 0);
  *blocks = n;
  *unused = n * block_size - tokens;
  return PA_OK;
}

pa_status pa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                       const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                       int32_t kv_heads, int32_t block_size, int32_t head_dim, int32_t dtype,
                       void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || kv_heads <= 0 || block_size <= 0 || head_dim <= 0 ||
      !dtype_ok(dtype))
    return PA_ERR_INVALID_ARG;
  const int64_t row_bytes = (int64_t)head_dim * elem_bytes(dtype);
  if (row_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_mapping, 8))
    return PA_ERR_INVALID_ARG;
  if ((int64_t)num_tokens * 2 * kv_heads * (row_bytes / 16) > (int64_t)INT32_MAX * 256)
    return PA_ERR_INVALID_ARG;
  return from_hip(pa::launch_kv_append(k_new, v_new, k_cache, v_cache, slot_mapping, num_tokens,
                                       num_blocks, kv_heads, block_size, (int)row_bytes,
                                       (int64_t)kv_heads * block_size * row_bytes,
                                       (hipStream_t)stream));
}

pa_status pa_decode_plan(int32_t num_seqs, int32_t num_heads, int32_t kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t max_seq_len, int32_t partition_size,
                         int32_t dtype, int32_t kernel, int32_t* kernel_used,
                         int32_t* eff_partition_size, int32_t* num_partitions,
                         size_t* workspace_bytes) {
  Plan plan;
  const pa_status st = make_plan(num_seqs, num_heads, kv_heads, head_dim, block_size,
                                 max_seq_len, partition_size, dtype, kernel, &plan);
  if (st != PA_OK) return st;
  if (kernel_used) *kernel_used = plan.kernel;
  if (eff_partition_size) *eff_partition_size = plan.partition;
  if (num_partitions) *num_partitions = plan.partitions;
  if (workspace_bytes) *workspace_bytes = plan.workspace;
  return PA_OK;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                                 int32_t partition_size, int32_t dtype) {
  Plan plan;
  if (make_plan(num_seqs, num_heads, kv_heads, head_dim, block_size, max_seq_len,
                partition_size, dtype, PA_KERNEL_AUTO, &plan) != PA_OK)
    return 0;
  return plan.workspace;
}

pa_status pa_decode_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* seq_lens, int32_t max_seq_len, int32_t num_seqs,
                       int32_t num_heads, int32_t kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, float scale,
                       int32_t partition_size, void* workspace, size_t workspace_bytes,
                       int32_t dtype, int32_t kernel, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                     max_seq_len, num_seqs, num_heads, kv_heads, head_dim, block_size,
                     num_blocks, scale, partition_size, workspace, workspace_bytes, dtype, kernel,
                     stream, nullptr, nullptr, nullptr);
}

pa_status pa_decode_ordered(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t max_seq_len, const int32_t* order,
                            int32_t num_seqs, int32_t num_heads, int32_t kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                            int32_t partition_size, void* workspace, size_t workspace_bytes,
                            int32_t dtype, int32_t kernel, void* stream) {
  if (order == nullptr && num_seqs > 0) return PA_ERR_INVALID_ARG;
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                     max_seq_len, num_seqs, num_heads, kv_heads, head_dim, block_size, num_blocks,
                     scale, partition_size, workspace, workspace_bytes, dtype, kernel, stream,
                     nullptr, nullptr, nullptr, nullptr, order);
}

pa_status pa_decode_append(void* out, const void* q, void* k_cache, void* v_cache,
                           const void* k_new, const void* v_new, const int64_t* slot_mapping,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t max_seq_len, int32_t num_seqs,
                           int32_t num_heads, int32_t kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, float scale,
                           int32_t partition_size, void* workspace, size_t workspace_bytes,
                           int32_t dtype, int32_t kernel, void* stream) {
  if (num_seqs > 0 && slot_mapping == nullptr) return PA_ERR_INVALID_ARG;
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                     max_seq_len, num_seqs, num_heads, kv_heads, head_dim, block_size,
                     num_blocks, scale, partition_size, workspace, workspace_bytes, dtype, kernel,
                     stream, k_new, v_new, num_seqs > 0 ? slot_mapping : nullptr);
}

pa_status pa_decode_append_ordered(void* out, const void* q, void* k_cache, void* v_cache,
                                   const void* k_new, const void* v_new,
                                   const int64_t* slot_mapping, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                   int32_t max_seq_len, const int32_t* order, int32_t num_seqs,
                                   int32_t num_heads, int32_t kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks, float scale,
                                   int32_t partition_size, void* workspace,
                                   size_t workspace_bytes, int32_t dtype, int32_t kernel,
                                   void* stream) {
  if (num_seqs > 0 && (slot_mapping == nullptr || order == nullptr)) return PA_ERR_INVALID_ARG;
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                     max_seq_len, num_seqs, num_heads, kv_heads, head_dim, block_size,
                     num_blocks, scale, partition_size, workspace, workspace_bytes, dtype, kernel,
                     stream, k_new, v_new, num_seqs > 0 ? slot_mapping : nullptr, nullptr,
                     order);
}

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t max_seq_len, int32_t num_seqs,
                    int32_t num_heads, int32_t kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t num_blocks, float scale, int32_t partition_size, void* workspace,
                    size_t workspace_bytes, int32_t dtype, void* stream) {
  return pa_decode_ex(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                      max_seq_len, num_seqs, num_heads, kv_heads, head_dim, block_size,
                      num_blocks, scale, partition_size, workspace, workspace_bytes, dtype,
                      PA_KERNEL_AUTO, stream);
}

pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t max_seq_len, int32_t num_seqs,
                            int32_t num_heads, int32_t kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, float scale,
                            int32_t partition_size, int32_t dtype, int32_t kernel,
                            void* stream) {
  Plan plan;
  const pa_status st = make_plan(num_seqs, num_heads, kv_heads, head_dim, block_size,
                                 max_seq_len, partition_size, dtype, kernel, &plan);
  if (st != PA_OK) return st;
  if (plan.workspace > kScratchBytes) return PA_ERR_SCRATCH;
  void* ws = nullptr;
  if (plan.workspace > 0 && num_seqs > 0) {
    ws = scratch_ptr();
    if (ws == nullptr) return PA_ERR_HIP;
  }
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                     max_seq_len, num_seqs, num_heads, kv_heads, head_dim, block_size,
                     num_blocks, scale, partition_size, ws, ws != nullptr ? kScratchBytes : 0,
                     dtype, kernel, stream, nullptr, nullptr, nullptr);
}

static pa_status shared_prefix_impl(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
    int32_t max_seq_len, int32_t num_seqs, int32_t num_heads, int32_t kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, float scale, const int32_t* group_start,
    const int32_t* group_prefix_blocks, int32_t num_groups, int32_t prefix_partition_size,
    int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t dtype, void* stream,
    const int32_t* order) {
  Plan plan;
  pa::PrefixGroups pg;
  const pa_status st = shared_prefix_plan(
      num_seqs, num_heads, kv_heads, head_dim, block_size, max_seq_len, max_blocks_per_seq,
      group_start, group_prefix_blocks, num_groups, prefix_partition_size, partition_size, dtype,
      &plan, &pg);
  if (st != PA_OK) return st;
  if (pg.num_groups == 0)  // nothing shared
    return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                       max_seq_len, num_seqs, num_heads, kv_heads, head_dim, block_size,
                       num_blocks, scale, partition_size, workspace, workspace_bytes, dtype,
                       PA_KERNEL_MFMA, stream, nullptr, nullptr, nullptr, nullptr, order);
  // the prefix kernel scales row maxima of raw scores, so scale must be > 0
  if (num_blocks <= 0 || !isfinite(scale) || !(scale > 0.0f)) return PA_ERR_INVALID_ARG;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens) return PA_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4))
    return PA_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < plan.workspace || !aligned(workspace, 16))
    return PA_ERR_INVALID_ARG;

  pa::DecodeParams p;
  memset(&p, 0, sizeof(p));
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.ws_o = (float*)workspace;
  p.ws_ml = p.ws_o + (size_t)num_seqs * num_heads * plan.partitions * head_dim;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.kv_heads = kv_heads;
  p.group = num_heads / kv_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_seq_len = max_seq_len;
  p.num_blocks = num_blocks;
  p.block_size = block_size;
  p.block_shift = log2i(block_size);
  p.partition_size = plan.partition;
  p.num_partitions = plan.partitions;
  p.waves = 4;  // the tail work-groups of the shared-prefix launch
  p.wave_parts = 0;
  p.scale_log2 = scale * 1.4426950408889634f;  // log2(e)
  p.num_layers = 1;
  p.prefix = pg;
  p.order = order;
  const hipStream_t s = (hipStream_t)stream;
  if (pa::launch_shared_prefix(p, head_dim, s) != hipSuccess) return PA_ERR_HIP;
  return from_hip(pa::launch_prefix_merge(p, head_dim, s));
}

pa_status pa_decode_shared_prefix(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                  int32_t max_seq_len, int32_t num_seqs, int32_t num_heads,
                                  int32_t kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, float scale, const int32_t* group_start,
                                  const int32_t* group_prefix_blocks, int32_t num_groups,
                                  int32_t prefix_partition_size, int32_t partition_size,
                                  void* workspace, size_t workspace_bytes, int32_t dtype,
                                  void* stream) {
  return shared_prefix_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                            max_seq_len, num_seqs, num_heads, kv_heads, head_dim, block_size,
                            num_blocks, scale, group_start, group_prefix_blocks, num_groups,
                            prefix_partition_size, partition_size, workspace, workspace_bytes,
                            dtype, stream, nullptr);
}

pa_status pa_decode_shared_prefix_ordered(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
    int32_t max_seq_len, const int32_t* order, int32_t num_seqs, int32_t num_heads,
    int32_t kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    const int32_t* group_start, const int32_t* group_prefix_blocks, int32_t num_groups,
    int32_t prefix_partition_size, int32_t partition_size, void* workspace,
    size_t workspace_bytes, int32_t dtype, void* stream) {
  if (order == nullptr && num_seqs > 0) return PA_ERR_INVALID_ARG;
  if (order != nullptr && !aligned(order, 4)) return PA_ERR_INVALID_ARG;
  return shared_prefix_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                            max_seq_len, num_seqs, num_heads, kv_heads, head_dim, block_size,
                            num_blocks, scale, group_start, group_prefix_blocks, num_groups,
                            prefix_partition_size, partition_size, workspace, workspace_bytes,
                            dtype, stream, order);
}

size_t pa_decode_shared_prefix_workspace_bytes(
    int32_t num_seqs, int32_t num_heads, int32_t kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_seq_len, int32_t max_blocks_per_seq, const int32_t* group_start,
    const int32_t* group_prefix_blocks, int32_t num_groups, int32_t prefix_partition_size,
    int32_t partition_size, int32_t dtype) {
  Plan plan;
  pa::PrefixGroups pg;
  if (shared_prefix_plan(num_seqs, num_heads, kv_heads, head_dim, block_size, max_seq_len,
                         max_blocks_per_seq, group_start, group_prefix_blocks, num_groups,
                         prefix_partition_size, partition_size, dtype, &plan, &pg) != PA_OK)
    return 0;
  return plan.workspace;
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                         int32_t num_pairs, int32_t num_blocks, int32_t kv_heads,
                         int32_t block_size, int32_t head_dim, int32_t dtype, void* stream) {
  if (num_pairs < 0 || num_blocks <= 0 || kv_heads <= 0 || block_size <= 0 || head_dim <= 0 ||
      !dtype_ok(dtype))
    return PA_ERR_INVALID_ARG;
  const int64_t block_bytes = (int64_t)kv_heads * block_size * head_dim * elem_bytes(dtype);
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_mapping, 8))
    return PA_ERR_INVALID_ARG;
  if ((int64_t)num_pairs * 2 * 64 > INT32_MAX) return PA_ERR_INVALID_ARG;
  return from_hip(pa::launch_move_blocks(k_cache, v_cache, num_blocks, k_cache, v_cache,
                                         num_blocks, block_mapping, num_pairs, block_bytes,
                                         (hipStream_t)stream));
}

pa_status pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* seq_lens, const int32_t* query_start, int32_t max_query_len,
                     int32_t num_seqs, int32_t num_queries, int32_t num_heads, int32_t kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                     int32_t dtype, void* stream) {
  if (num_seqs < 0 || num_queries < 0 || max_query_len < 0 || num_heads <= 0 || kv_heads <= 0 ||
      num_heads % kv_heads != 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || !dtype_ok(dtype) || !isfinite(scale) || !(scale > 0.0f))
    return PA_ERR_INVALID_ARG;
  const int32_t group = num_heads / kv_heads;
  // the matrix-core kernel for bf16 at block sizes >= 16, the vector-ALU one
  // for fp32 and smaller blocks
  const bool mfma = dtype == PA_BF16 && (head_dim == 64 || head_dim == 128) &&
                    pow2(block_size) && block_size >= 16 && block_size <= 256 && pow2(group) &&
                    group <= 16;
  const bool valu = valu_supports(dtype, head_dim, group, block_size);
  if (!mfma && !valu) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_queries == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start)
    return PA_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(query_start, 4))
    return PA_ERR_INVALID_ARG;
  const int64_t q_tiles = ceil_div((int64_t)max_query_len * group, pa::kPrefillRows);
  const int64_t pairs8 = round_up((int64_t)num_seqs * kv_heads, 8);
  if (pairs8 * q_tiles > INT32_MAX) return PA_ERR_INVALID_ARG;
  if (!mfma && ceil_div(max_query_len, pa::kPrefillValuRows) * num_seqs * kv_heads > INT32_MAX)
    return PA_ERR_INVALID_ARG;

  pa::PrefillParams p;
  memset(&p, 0, sizeof(p));
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.query_start = query_start;
  p.num_seqs = num_seqs;
  p.num_queries = num_queries;
  p.max_query_len = max_query_len;
  p.num_heads = num_heads;
  p.kv_heads = kv_heads;
  p.group = group;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.block_size = block_size;
  p.block_shift = log2i(block_size);
  p.q_tiles = (int32_t)q_tiles;
  p.scale_log2 = scale * 1.4426950408889634f;  // log2(e)
  if (!mfma)
    return from_hip(pa::launch_prefill_valu(p, dtype == PA_BF16, head_dim, (hipStream_t)stream));
  return from_hip(pa::launch_prefill_mfma(p, head_dim, (hipStream_t)stream));
}

pa_status pa_swap_blocks(void* dst_k, void* dst_v, int64_t dst_num_blocks, const void* src_k,
                         const void* src_v, int64_t src_num_blocks, const int64_t* block_mapping,
                         int32_t num_pairs, int32_t kv_heads, int32_t block_size,
                         int32_t head_dim, int32_t dtype, void* stream) {
  if (num_pairs < 0 || dst_num_blocks <= 0 || src_num_blocks <= 0 || kv_heads <= 0 ||
      block_size <= 0 || head_dim <= 0 || !dtype_ok(dtype))
    return PA_ERR_INVALID_ARG;
  const int64_t block_bytes = (int64_t)kv_heads * block_size * head_dim * elem_bytes(dtype);
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if ((int64_t)num_pairs * 2 * 64 > INT32_MAX) return PA_ERR_INVALID_ARG;
  const void* p[5] = {dst_k, dst_v, src_k, src_v, block_mapping};
  const void* kp[5];
  Residency r[5];
  for (int i = 0; i < 5; ++i) {
    r[i] = residency(p[i], &kp[i]);
    if (r[i] == kUnknown || !aligned(kp[i], i == 4 ? 8 : 16)) return PA_ERR_INVALID_ARG;
  }
  // the two caches of a pool live together; host-to-host moves are not GPU work
  if (r[0] != r[1] || r[2] != r[3]) return PA_ERR_INVALID_ARG;
  if (r[0] == kPinnedHost && r[2] == kPinnedHost) return PA_ERR_UNSUPPORTED;
  return from_hip(pa::launch_move_blocks((void*)kp[0], (void*)kp[1], dst_num_blocks, kp[2], kp[3],
                                         src_num_blocks, (const int64_t*)kp[4], num_pairs,
                                         block_bytes, (hipStream_t)stream));
}

// ---- layered pool: [num_blocks][2][num_layers][kv_heads][block_size][head_dim] ----

static bool layered_args_ok(int32_t num_layers, int32_t kv_heads, int32_t block_size,
                            int32_t head_dim) {
  return num_layers > 0 && kv_heads > 0 && block_size > 0 && head_dim > 0;
}

pa_status pa_kv_append_layered(const void* k_new, const void* v_new, void* kv_pool, int32_t layer,
                               int32_t num_layers, const int64_t* slot_mapping,
                               int32_t num_tokens, int32_t num_blocks, int32_t kv_heads,
                               int32_t block_size, int32_t head_dim, int32_t dtype,
                               void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || !layered_args_ok(num_layers, kv_heads, block_size,
                                                             head_dim) ||
      layer < 0 || layer >= num_layers || !dtype_ok(dtype))
    return PA_ERR_INVALID_ARG;
  const int64_t row_bytes = (int64_t)head_dim * elem_bytes(dtype);
  if (row_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !kv_pool || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(kv_pool, 16) ||
      !aligned(slot_mapping, 8))
    return PA_ERR_INVALID_ARG;
  if ((int64_t)num_tokens * 2 * kv_heads * (row_bytes / 16) > (int64_t)INT32_MAX * 256)
    return PA_ERR_INVALID_ARG;
  const int64_t layer_bytes = (int64_t)kv_heads * block_size * row_bytes;
  char* base = (char*)kv_pool;
  return from_hip(pa::launch_kv_append(k_new, v_new, base + layer * layer_bytes,
                                       base + ((int64_t)num_layers + layer) * layer_bytes,
                                       slot_mapping, num_tokens, num_blocks, kv_heads, block_size,
                                       (int)row_bytes, 2 * num_layers * layer_bytes,
                                       (hipStream_t)stream));
}

pa_status pa_decode_layered(void* out, const void* q, const void* kv_pool, int32_t first_layer,
                            int32_t layers, int32_t num_layers, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens,
                            int32_t max_seq_len, int32_t num_seqs, int32_t num_heads,
                            int32_t kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, float scale, int32_t partition_size,
                            void* workspace, size_t workspace_bytes, int32_t dtype,
                            void* stream) {
  if (!layered_args_ok(num_layers, kv_heads, block_size, head_dim) || layers <= 0 ||
      first_layer < 0 || first_layer + (int64_t)layers > num_layers || layers > 65535)
    return PA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return PA_ERR_INVALID_ARG;
  const int64_t layer_elems = (int64_t)kv_heads * block_size * head_dim;
  const char* base = (const char*)kv_pool;
  const int64_t eb = elem_bytes(dtype);
  LayerSpec lay;
  lay.block_stride = 2 * num_layers * layer_elems;
  lay.layer_kv_stride = layer_elems;
  lay.layers = layers;
  const void* k = kv_pool ? base + first_layer * layer_elems * eb : nullptr;
  const void* v = kv_pool ? base + ((int64_t)num_layers + first_layer) * layer_elems * eb : nullptr;
  return decode_impl(out, q, k, v, block_tables, max_blocks_per_seq, seq_lens, max_seq_len,
                     num_seqs, num_heads, kv_heads, head_dim, block_size, num_blocks, scale,
                     partition_size, workspace, workspace_bytes, dtype, PA_KERNEL_AUTO, stream,
                     nullptr, nullptr, nullptr, &lay);
}

pa_status pa_copy_blocks_layered(void* kv_pool, const int64_t* block_mapping, int32_t num_pairs,
                                 int32_t num_blocks, int32_t num_layers, int32_t kv_heads,
                                 int32_t block_size, int32_t head_dim, int32_t dtype,
                                 void* stream) {
  if (num_pairs < 0 || num_blocks <= 0 ||
      !layered_args_ok(num_layers, kv_heads, block_size, head_dim) || !dtype_ok(dtype))
    return PA_ERR_INVALID_ARG;
  const int64_t block_bytes =
      2 * (int64_t)num_layers * kv_heads * block_size * head_dim * elem_bytes(dtype);
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!kv_pool || !block_mapping || !aligned(kv_pool, 16) || !aligned(block_mapping, 8))
    return PA_ERR_INVALID_ARG;
  if ((int64_t)num_pairs * 64 > INT32_MAX) return PA_ERR_INVALID_ARG;
  return from_hip(pa::launch_move_blocks(kv_pool, nullptr, num_blocks, kv_pool, nullptr,
                                         num_blocks, block_mapping, num_pairs, block_bytes,
                                         (hipStream_t)stream));
}

pa_status pa_swap_blocks_layered(void* dst_pool, int64_t dst_num_blocks, const void* src_pool,
                                 int64_t src_num_blocks, const int64_t* block_mapping,
                                 int32_t num_pairs, int32_t num_layers, int32_t kv_heads,
                                 int32_t block_size, int32_t head_dim, int32_t dtype,
                                 void* stream) {
  if (num_pairs < 0 || dst_num_blocks <= 0 || src_num_blocks <= 0 ||
      !layered_args_ok(num_layers, kv_heads, block_size, head_dim) || !dtype_ok(dtype))
    return PA_ERR_INVALID_ARG;
  const int64_t block_bytes =
      2 * (int64_t)num_layers * kv_heads * block_size * head_dim * elem_bytes(dtype);
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if ((int64_t)num_pairs * 64 > INT32_MAX) return PA_ERR_INVALID_ARG;
  const void* p[3] = {dst_pool, src_pool, block_mapping};
  const void* kp[3];
  Residency r[3];
  for (int i = 0; i < 3; ++i) {
    r[i] = residency(p[i], &kp[i]);
    if (r[i] == kUnknown || !aligned(kp[i], i == 2 ? 8 : 16)) return PA_ERR_INVALID_ARG;
  }
  if (r[0] == kPinnedHost && r[1] == kPinnedHost) return PA_ERR_UNSUPPORTED;
  return from_hip(pa::launch_move_blocks((void*)kp[0], nullptr, dst_num_blocks, kp[1], nullptr,
                                         src_num_blocks, (const int64_t*)kp[2], num_pairs,
                                         block_bytes, (hipStream_t)stream));
}

}  // extern "C"
