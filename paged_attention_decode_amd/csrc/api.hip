// Host side of libpagedattn: argument checks, launch planning, workspace and
// the extern "C" entry points declared in include/pagedattn.h.

#include "pa_internal.h"
#include "pagedattn.h"

#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <climits>
#include <mutex>
#include <string>

namespace {

using namespace pa;

thread_local std::string t_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  t_error = buf;
  return code;
}

int ok() {
  t_error.clear();
  return PA_OK;
}

// Attention-kernel workgroups per compute unit that one call plans for.
// Ranges are sized for this many resident wavefronts (4 per workgroup).
#ifndef PA_GROUPS_PER_CU
#define PA_GROUPS_PER_CU 2
#endif
constexpr int kGroupsPerCU = PA_GROUPS_PER_CU;
#ifndef PA_PREFILL_SHARED
#define PA_PREFILL_SHARED 1
#endif
constexpr bool kPrefillShared = PA_PREFILL_SHARED != 0;
// partition_size values: 0 automatic, -1 one pass, -2 balanced ranges, -3 workgroup split,
// > 0 fixed ranges.
constexpr int kBalanced = -2;
constexpr int64_t kOnePassMaxTokens = 512;

struct DeviceState {
  bool init = false;
  int num_cus = 0;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  // Device address of this device's copy of `scratch` (below), once looked up.
  void* scratch_ptr = nullptr;
};

// Fixed storage, so a DeviceState pointer stays valid while other threads
// initialise further devices.
constexpr int kMaxDevices = 64;
std::mutex g_mutex;
DeviceState g_devices[kMaxDevices];

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int ilog2(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct Plan {
  int64_t num_waves = 0;
  int64_t num_ranges = 0;  // ranges the workspace has rows for (split modes)
  int grid = 0;
  int range_tiles = 0;  // -1 one pass, kWorkgroupSplit, 0 balanced, >0 fixed
  bool reduce = false;
  size_t lds = 0;
  int n_hg = 0, gh_max = 0, segs_per_seq = 0;
  int casc_width = 0;  // shared-prefix window (0: off)
  int ws_cols = 0;     // partial-output columns per (range, slot)
  int stash_slots = 0, stash_slot_floats = 0, stash_off = 0;  // deferred rows (split modes)
  int64_t whole_own_row = 0, whole_pre_row = 0;
  size_t off_lse = 0, off_meta = 0, off_meta_pre = 0, off_share = 0, ws_bytes = 0;
};

bool valid_dtype(int dt) { return dt == PA_DTYPE_F32 || dt == PA_DTYPE_F16 || dt == PA_DTYPE_BF16; }

int check_decode_sizes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t max_blocks, int32_t dtype, int32_t partition_size) {
  if (!valid_dtype(dtype)) return fail(PA_ERR_DTYPE, "dtype %d is not one of PA_DTYPE_F32/F16/BF16", dtype);
  if (num_seqs < 0) return fail(PA_ERR_SHAPE, "num_seqs %d < 0", num_seqs);
  if (num_seqs > kMaxSeqs) return fail(PA_ERR_UNSUPPORTED, "num_seqs %d exceeds %d", num_seqs, kMaxSeqs);
  if (num_heads <= 0 || num_kv_heads <= 0)
    return fail(PA_ERR_SHAPE, "num_heads %d and num_kv_heads %d must be positive", num_heads, num_kv_heads);
  if (num_heads % num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "num_heads %d is not a multiple of num_kv_heads %d", num_heads, num_kv_heads);
  if (head_dim <= 0) return fail(PA_ERR_SHAPE, "head_dim %d must be positive", head_dim);
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128, 256)", head_dim);
  if (block_size <= 0) return fail(PA_ERR_SHAPE, "block_size %d must be positive", block_size);
  if (!is_pow2(block_size) || block_size < 16 || block_size > 256)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not supported (power of two in [16, 256])", block_size);
  if (max_blocks <= 0) return fail(PA_ERR_SHAPE, "max_blocks_per_seq %d must be positive", max_blocks);
  if ((int64_t)max_blocks * block_size > INT32_MAX / 2)
    return fail(PA_ERR_UNSUPPORTED, "max_blocks_per_seq * block_size too large");
  if (partition_size < kWorkgroupSplit || (partition_size > 0 && partition_size % kTile != 0))
    return fail(PA_ERR_SHAPE, "partition_size %d must be -3, -2, -1, 0 or a positive multiple of 16", partition_size);
  return PA_OK;
}

int make_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
              int32_t max_blocks, int32_t partition_size, bool shared_prefix, int num_cus, Plan* p) {
  const int group = num_heads / num_kv_heads;
  p->n_hg = (group + kHeadsPerTile - 1) / kHeadsPerTile;
  p->gh_max = group < kHeadsPerTile ? group : kHeadsPerTile;
  p->segs_per_seq = num_kv_heads * p->n_hg;
  const int64_t segs = (int64_t)num_seqs * p->segs_per_seq;
  const int64_t max_tiles = ((int64_t)max_blocks * block_size + kTile - 1) / kTile;
  const int64_t upper_tiles = segs * (max_tiles > 0 ? max_tiles : 1);
  const int64_t resident = (int64_t)num_cus * kGroupsPerCU * kWavesPerGroup;
  int64_t waves;
  // Automatic: when no context can be longer than kOnePassMaxTokens (the host's bound,
  // max_blocks * block_size; it reads no device memory) every segment is short and no merge
  // kernel is needed. Then, if every segment gets a resident workgroup of its own, the workgroup
  // split puts four wavefronts on each segment's chain of dependent loads; with more segments
  // one wavefront per segment (one pass), since the split would leave three of four wavefronts
  // idle on one-tile segments. Otherwise balanced ranges.
  if (partition_size == 0) {
    if ((int64_t)max_blocks * block_size <= kOnePassMaxTokens)
      partition_size = segs <= resident / kWavesPerGroup ? kWorkgroupSplit : -1;
    else
      partition_size = kBalanced;
  }
  // Workgroup split keeps four partial outputs and their log-sum-exps in LDS; where they would
  // not fit in 64 KiB (head_dim 256 with 16 heads per group) it runs as one pass.
  const size_t split_lds = (size_t)kWavesPerGroup * p->gh_max * (head_dim + 1) * sizeof(float);
  if (partition_size == kWorkgroupSplit && split_lds > 65536) partition_size = -1;
  if (partition_size == kWorkgroupSplit) {
    // One workgroup per segment (persistent when there are more segments than resident groups).
    p->range_tiles = kWorkgroupSplit;
    const int64_t groups = resident / kWavesPerGroup;
    waves = (segs < groups ? segs : groups) * kWavesPerGroup;
    p->lds = split_lds;
    p->reduce = false;
  } else if (partition_size == -1) {
    p->range_tiles = -1;
    waves = segs < resident ? segs : resident;
    p->lds = 0;
    p->reduce = false;
  } else {
    if (upper_tiles + max_tiles >= INT32_MAX / 2)
      return fail(PA_ERR_UNSUPPORTED, "batch too large: %lld tiles", (long long)upper_tiles);
    p->lds = (size_t)(num_seqs + 1) * sizeof(int32_t);
    p->reduce = true;
    if (partition_size == kBalanced) {
      // One range per wavefront, sized on the device from the actual lengths.
      p->range_tiles = 0;
      const int64_t useful = (upper_tiles + kMinTilesPerWave - 1) / kMinTilesPerWave;
      waves = useful < resident ? useful : resident;
    } else {
      // Fixed ranges: the lengths live on the device, so the workspace has rows for the
      // ranges of the longest possible batch, and the resident wavefronts loop over the
      // ranges the actual lengths need.
      p->range_tiles = partition_size / kTile;
      p->num_ranges = (upper_tiles + p->range_tiles - 1) / p->range_tiles;
      waves = p->num_ranges < resident ? p->num_ranges : resident;
    }
  }
  if (waves < 1) waves = 1;
  p->grid = (int)((waves + kWavesPerGroup - 1) / kWavesPerGroup);
  p->num_waves = (int64_t)p->grid * kWavesPerGroup;
  // Shared prefixes need the split modes' merge, two or more sequences' head groups per
  // 16-column tile, and the sharing words in LDS beside the prefix sums.
  p->casc_width = 0;
  p->ws_cols = p->gh_max;
  if (shared_prefix && p->reduce && p->n_hg == 1 && kHeadsPerTile / group >= 2 && num_seqs <= kMaxSharedSeqs) {
    p->casc_width = kHeadsPerTile / group;
    p->ws_cols = kHeadsPerTile;
    p->lds += (size_t)num_seqs * sizeof(int32_t);
  }
  if (p->reduce) {
    // Deferred rows: on gfx9-family GPUs a store counts in the same wait counter as the loads,
    // so every later tile wait would also wait for the store to be acknowledged, which takes
    // long under a full read stream. A wavefront therefore keeps the rows of its pieces in LDS
    // slots after the prefix sums (header of 16 words, ws_cols rows of head_dim floats, their
    // lse values) and writes them after its last tile; with no slot free it writes at once.
    const size_t base = (p->lds + 15) & ~size_t(15);
    const size_t slot_floats = 16 + (size_t)p->ws_cols * head_dim + (((size_t)p->ws_cols + 3) & ~size_t(3));
    const size_t per_slot = (size_t)kWavesPerGroup * slot_floats * sizeof(float);
    size_t slots = base < (size_t)kStashLdsBytes ? ((size_t)kStashLdsBytes - base) / per_slot : 0;
    if (slots > (size_t)kMaxStashSlots) slots = kMaxStashSlots;
    p->stash_slots = (int)slots;
    p->stash_slot_floats = (int)slot_floats;
    p->stash_off = (int)(base / sizeof(float));
    if (slots > 0) p->lds = base + slots * per_slot;
    if (p->range_tiles == 0 || p->num_ranges < p->num_waves) p->num_ranges = p->num_waves;
    const size_t windows = p->casc_width > 0 ? ((size_t)num_seqs + p->casc_width - 1) / p->casc_width : 0;
    // Rows of pieces cut by range boundaries; with shared prefixes also rows for whole segments
    // that are merged with a prefix (own segments of group members, and prefix segments).
    p->whole_own_row = (int64_t)p->num_ranges * 2 * p->ws_cols;
    p->whole_pre_row = p->whole_own_row + (p->casc_width > 0 ? segs * p->gh_max : 0);
    const size_t rows = (size_t)p->whole_pre_row + windows * p->segs_per_seq * kHeadsPerTile;
    p->off_lse = align256(rows * head_dim * sizeof(float));
    p->off_meta = p->off_lse + align256(rows * sizeof(float));
    p->ws_bytes = p->off_meta + align256((size_t)segs * sizeof(int4));
    if (p->casc_width > 0) {
      p->off_meta_pre = p->ws_bytes;
      p->off_share = p->off_meta_pre + align256(windows * p->segs_per_seq * sizeof(int4));
      p->ws_bytes = p->off_share + align256((size_t)num_seqs * sizeof(int32_t));
    }
  } else {
    p->off_lse = p->off_meta = p->ws_bytes = 0;
  }
  return PA_OK;
}

int device_state(DeviceState** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mutex);
  DeviceState& st = g_devices[dev];
  if (!st.init) {
    int cus = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || cus <= 0) return fail(PA_ERR_HIP, "cannot query compute units: %s", hipGetErrorString(e));
    st.num_cus = cus;
    st.init = true;
  }
  *out = &st;
  return PA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workspace of pa_paged_attention_decode_noalloc: fixed device memory, one copy per device,
// held until the process ends. In host code `scratch` names a host-side stand-in, not device
// memory: host code uses only the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

// Looks up (once per device, with that device current) the device address of `scratch`.
int scratch_address(DeviceState* st, void** out) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!st->scratch_ptr) {
    void* ptr = nullptr;
    hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !ptr)
      return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(err));
    st->scratch_ptr = ptr;
  }
  *out = st->scratch_ptr;
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_store_kvcache(const void* k, const void* v, const int32_t* slot_mapping, void* k_cache, void* v_cache,
                     int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int64_t num_blocks, int64_t k_token_stride, int64_t v_token_stride, int32_t dtype,
                     void* stream) {
  if (!valid_dtype(dtype)) return fail(PA_ERR_DTYPE, "dtype %d is not one of PA_DTYPE_F32/F16/BF16", dtype);
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens %d < 0", num_tokens);
  const int e = elem_bytes(dtype);
  const int x = 16 / e;
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_SHAPE, "num_kv_heads %d, head_dim %d, block_size %d, num_blocks %lld must be positive",
                num_kv_heads, head_dim, block_size, (long long)num_blocks);
  if (head_dim % x != 0 || head_dim > 1024)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d must be a multiple of %d and at most 1024", head_dim, x);
  if (block_size % 4 != 0) return fail(PA_ERR_UNSUPPORTED, "block_size %d must be a multiple of 4", block_size);
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return fail(PA_ERR_NULL, "a required pointer is NULL");
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (k_token_stride < row || v_token_stride < row)
    return fail(PA_ERR_SHAPE, "token strides (%lld, %lld) smaller than num_kv_heads*head_dim %lld",
                (long long)k_token_stride, (long long)v_token_stride, (long long)row);
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (k_token_stride * e) % 16 != 0 || (v_token_stride * e) % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "k, v and the caches must be 16-byte aligned with 16-byte token strides");
  if ((int64_t)num_tokens * num_kv_heads * (head_dim / x) > (int64_t)INT32_MAX * 256)
    return fail(PA_ERR_UNSUPPORTED, "too many tokens");
  StoreArgs a;
  a.k = k;
  a.v = v;
  a.slot_mapping = slot_mapping;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_stride = k_token_stride;
  a.v_stride = v_token_stride;
  a.num_slots = num_blocks * block_size;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  hipError_t err = launch_store(a, dtype, reinterpret_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(PA_ERR_HIP, "store_kvcache launch failed: %s", hipGetErrorString(err));
  return ok();
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst, int32_t num_pairs,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t dtype,
                   void* stream) {
  if (!valid_dtype(dtype)) return fail(PA_ERR_DTYPE, "dtype %d is not one of PA_DTYPE_F32/F16/BF16", dtype);
  if (num_pairs < 0) return fail(PA_ERR_SHAPE, "num_pairs %d < 0", num_pairs);
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_SHAPE, "num_kv_heads, head_dim, block_size and num_blocks must be positive");
  const int e = elem_bytes(dtype);
  const int64_t block_bytes = (int64_t)num_kv_heads * head_dim * block_size * e;
  if (block_bytes % 16 != 0) return fail(PA_ERR_UNSUPPORTED, "block bytes must be a multiple of 16");
  if (num_pairs == 0) return ok();
  if (!k_cache || !v_cache || !src || !dst) return fail(PA_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(k_cache) || !aligned16(v_cache)) return fail(PA_ERR_UNSUPPORTED, "caches must be 16-byte aligned");
  hipError_t err = launch_copy_blocks(k_cache, v_cache, src, dst, num_pairs, block_bytes, num_blocks,
                                      reinterpret_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(PA_ERR_HIP, "copy_blocks launch failed: %s", hipGetErrorString(err));
  return ok();
}

int pa_paged_prefill(const void* q, int64_t q_token_stride, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                     float scale, void* out, int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                     int64_t num_blocks, int32_t dtype, int32_t out_dtype, void* stream) {
  int rc = check_decode_sizes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, dtype, 0);
  if (rc != PA_OK) return rc;
  if (!valid_dtype(out_dtype) || (out_dtype != PA_DTYPE_F32 && out_dtype != dtype))
    return fail(PA_ERR_DTYPE, "out_dtype %d must be PA_DTYPE_F32 or the input dtype %d", out_dtype, dtype);
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens %d < 0", num_tokens);
  if (num_blocks <= 0) return fail(PA_ERR_SHAPE, "num_blocks %lld must be positive", (long long)num_blocks);
  if (q_token_stride < (int64_t)num_heads * head_dim)
    return fail(PA_ERR_SHAPE, "q_token_stride %lld smaller than num_heads*head_dim", (long long)q_token_stride);
  if (num_seqs == 0 || num_tokens == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  const int e = elem_bytes(dtype);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      (q_token_stride * e) % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "q, the caches and out must be 16-byte aligned (q rows too)");
  DeviceState* st = nullptr;
  rc = device_state(&st);
  if (rc != PA_OK) return rc;
  PrefillArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_tokens = num_tokens;
  a.out = out;
  a.q_token_stride = q_token_stride;
  a.num_blocks = num_blocks;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.n_hg = (a.group + kHeadsPerTile - 1) / kHeadsPerTile;
  a.gh_max = a.group < kHeadsPerTile ? a.group : kHeadsPerTile;
  a.block_size = block_size;
  a.bs_log2 = ilog2(block_size);
  a.max_blocks = max_blocks_per_seq;
  a.out_f32 = out_dtype == PA_DTYPE_F32 ? 1 : 0;
  // Each call takes the next set of work-queue counters, so calls that overlap on one device
  // (other streams) use different counters unless kQueueSlots of them are in flight at once.
  static std::atomic<uint32_t> calls{0};
  a.queue_slot = (int32_t)(calls.fetch_add(1, std::memory_order_relaxed) % kQueueSlots);
  const int qpi = prefill_queries_per_item(dtype, head_dim, a.gh_max);
  const size_t prefix_bytes = (size_t)((num_seqs + 1 + 3) & ~3) * sizeof(int32_t);
  hipError_t err;
  // 16-bit inputs at head_dim 128: four wavefronts share each K/V step through LDS (a quarter of
  // the L2 traffic, which bounds the per-wavefront kernel there). At head_dim 64 the per-wavefront
  // kernel is bound by its arithmetic instead and is faster; it also serves fp32, head_dim 256,
  // and batches whose item prefix would push the shared kernel's LDS past 64 KiB.
  const size_t shared_lds = prefix_bytes + prefill_shared_buffer_bytes(head_dim);
  if (kPrefillShared && dtype != PA_DTYPE_F32 && head_dim == 128 && shared_lds <= 65536) {
    const int wq = kWavesPerGroup * qpi;
    const int64_t items = (int64_t)num_kv_heads * a.n_hg * (((int64_t)num_tokens + wq - 1) / wq + num_seqs);
    const int64_t resident = (int64_t)st->num_cus * kGroupsPerCU;
    int64_t grid = items < resident ? items : resident;
    if (grid < 1) grid = 1;
    a.num_waves = (int)grid * kWavesPerGroup;
    err = launch_prefill_shared(a, dtype, head_dim, (int)grid, shared_lds, reinterpret_cast<hipStream_t>(stream));
  } else {
    const int64_t items = (int64_t)num_kv_heads * a.n_hg * (((int64_t)num_tokens + qpi - 1) / qpi + num_seqs);
    const int64_t resident = (int64_t)st->num_cus * kGroupsPerCU * kWavesPerGroup;
    int64_t waves = items < resident ? items : resident;
    if (waves < 1) waves = 1;
    const int grid = (int)((waves + kWavesPerGroup - 1) / kWavesPerGroup);
    a.num_waves = grid * kWavesPerGroup;
    err = launch_prefill(a, dtype, head_dim, grid, (size_t)(num_seqs + 1) * sizeof(int32_t),
                         reinterpret_cast<hipStream_t>(stream));
  }
  if (err != hipSuccess) return fail(PA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(err));
  return ok();
}

int pa_decode_plan_ex(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t max_blocks_per_seq, int32_t dtype, const pa_decode_opts* opts,
                      int32_t num_cus, int64_t* num_waves, int32_t* range_tokens, int32_t* uses_reduce,
                      int32_t* shared_prefix_window, size_t* workspace_bytes) {
  const int32_t partition_size = opts ? opts->partition_size : 0;
  int rc = check_decode_sizes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, dtype,
                              partition_size);
  if (rc != PA_OK) return rc;
  if (num_cus <= 0) {
    DeviceState* st = nullptr;
    rc = device_state(&st);
    if (rc != PA_OK) return rc;
    num_cus = st->num_cus;
  }
  Plan p;
  rc = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, partition_size,
                 opts && opts->shared_prefix != 0, num_cus, &p);
  if (rc != PA_OK) return rc;
  if (num_waves) *num_waves = p.num_waves;
  if (range_tokens) *range_tokens = p.range_tiles > 0 ? p.range_tiles * kTile : p.range_tiles;
  if (uses_reduce) *uses_reduce = p.reduce ? 1 : 0;
  if (shared_prefix_window) *shared_prefix_window = p.casc_width;
  if (workspace_bytes) *workspace_bytes = p.ws_bytes;
  return ok();
}

int pa_decode_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int32_t max_blocks_per_seq, int32_t dtype, int32_t partition_size, int32_t num_cus,
                   int64_t* num_waves, int32_t* range_tokens, int32_t* uses_reduce, size_t* workspace_bytes) {
  pa_decode_opts o = {};
  o.partition_size = partition_size;
  return pa_decode_plan_ex(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, dtype, &o,
                           num_cus, num_waves, range_tokens, uses_reduce, nullptr, workspace_bytes);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_blocks_per_seq, int32_t dtype,
                                 int32_t partition_size) {
  size_t bytes = 0;
  if (pa_decode_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, dtype,
                     partition_size, 0, nullptr, nullptr, nullptr, &bytes) != PA_OK)
    return 0;
  return bytes;
}

}  // extern "C"

namespace {

// Shared body of the decode entry points; k_new/v_new non-null = fused scatter of the step's token.
int decode_impl(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                const int32_t* context_lens, float scale, void* out, int32_t num_seqs, int32_t num_heads,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                int64_t num_blocks, int64_t q_seq_stride, int32_t dtype, int32_t out_dtype,
                const pa_decode_opts* opts, void* stream, const void* k_new, const void* v_new,
                int64_t k_new_stride, int64_t v_new_stride, bool noalloc = false) {
  const int32_t psize = opts ? opts->partition_size : 0;
  if (noalloc && opts && opts->workspace)
    return fail(PA_ERR_WORKSPACE, "the no-allocation entry point uses its fixed scratch; opts->workspace must be NULL");
  int rc = check_decode_sizes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, dtype,
                              psize);
  if (rc != PA_OK) return rc;
  if (!valid_dtype(out_dtype) || (out_dtype != PA_DTYPE_F32 && out_dtype != dtype))
    return fail(PA_ERR_DTYPE, "out_dtype %d must be PA_DTYPE_F32 or the input dtype %d", out_dtype, dtype);
  if (num_blocks <= 0) return fail(PA_ERR_SHAPE, "num_blocks %lld must be positive", (long long)num_blocks);
  if (q_seq_stride < (int64_t)num_heads * head_dim)
    return fail(PA_ERR_SHAPE, "q_seq_stride %lld smaller than num_heads*head_dim", (long long)q_seq_stride);
  if (num_seqs == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  const int e = elem_bytes(dtype);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      (q_seq_stride * e) % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "q, the caches and out must be 16-byte aligned (q rows too)");

  DeviceState* st = nullptr;
  rc = device_state(&st);
  if (rc != PA_OK) return rc;
  Plan p;
  rc = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, psize,
                 opts && opts->shared_prefix != 0, st->num_cus, &p);
  if (rc != PA_OK) return rc;

  char* ws = nullptr;
  if (p.ws_bytes > 0) {
    if (noalloc) {
      if (p.ws_bytes > (size_t)PA_NOALLOC_SCRATCH_BYTES)
        return fail(PA_ERR_WORKSPACE,
                    "this call's plan needs %zu bytes of workspace, more than the %zu-byte fixed scratch of "
                    "pa_paged_attention_decode_noalloc",
                    p.ws_bytes, (size_t)PA_NOALLOC_SCRATCH_BYTES);
      void* sp = nullptr;
      rc = scratch_address(st, &sp);
      if (rc != PA_OK) return rc;
      ws = reinterpret_cast<char*>(sp);
    } else if (opts && opts->workspace) {
      if (opts->workspace_bytes < p.ws_bytes)
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", opts->workspace_bytes, p.ws_bytes);
      if ((reinterpret_cast<uintptr_t>(opts->workspace) & 255u) != 0)
        return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
      ws = reinterpret_cast<char*>(opts->workspace);
    } else {
      std::lock_guard<std::mutex> lock(g_mutex);
      if (st->ws_bytes < p.ws_bytes) {
        if (st->ws) {
          (void)hipFree(st->ws);
          st->ws = nullptr;
          st->ws_bytes = 0;
        }
        void* mem = nullptr;
        hipError_t err = hipMalloc(&mem, p.ws_bytes);
        if (err != hipSuccess)
          return fail(PA_ERR_HIP, "workspace allocation of %zu bytes failed: %s", p.ws_bytes, hipGetErrorString(err));
        st->ws = mem;
        st->ws_bytes = p.ws_bytes;
      }
      ws = reinterpret_cast<char*>(st->ws);
    }
  }

  DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.ws_o = ws ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_lse = ws ? reinterpret_cast<float*>(ws + p.off_lse) : nullptr;
  a.ws_meta = ws ? reinterpret_cast<int4*>(ws + p.off_meta) : nullptr;
  a.ws_meta_pre = (ws && p.casc_width > 0) ? reinterpret_cast<int4*>(ws + p.off_meta_pre) : nullptr;
  a.ws_share = (ws && p.casc_width > 0) ? reinterpret_cast<int32_t*>(ws + p.off_share) : nullptr;
  a.ws_cols = p.ws_cols;
  a.stash_slots = p.stash_slots;
  a.stash_slot_floats = p.stash_slot_floats;
  a.stash_off = p.stash_off;
  a.whole_own_row = p.whole_own_row;
  a.whole_pre_row = p.whole_pre_row;
  // A prefix piece addresses the query rows of a whole window from one buffer resource.
  a.casc_width = ((int64_t)p.casc_width * q_seq_stride * e < INT32_MAX) ? p.casc_width : 0;
  a.q_seq_stride = q_seq_stride;
  a.num_blocks = num_blocks;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.n_hg = p.n_hg;
  a.gh_max = p.gh_max;
  a.segs_per_seq = p.segs_per_seq;
  a.block_size = block_size;
  a.bs_log2 = ilog2(block_size);
  a.max_blocks = max_blocks_per_seq;
  a.out_f32 = out_dtype == PA_DTYPE_F32 ? 1 : 0;
  a.num_waves = (int32_t)p.num_waves;
  a.range_tiles = p.range_tiles;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_new_stride = k_new_stride;
  a.v_new_stride = v_new_stride;
  {
    const int32_t hint = opts ? opts->cached_prefix_tokens : 0;
    a.cached_prefix_tokens = hint == 0 ? PA_DEFAULT_CACHED_PREFIX_TOKENS : (hint < 0 ? 0 : hint);
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // Fused step where the attention kernel does not take the token itself: the token is written to
  // its cache slot first, and the plain kernels run (neither writes the slot again).
  if (a.k_new != nullptr && !decode_fuses_step(dtype, head_dim)) {
    hipError_t err = launch_append(a, dtype, head_dim, s);
    if (err != hipSuccess) return fail(PA_ERR_HIP, "token append launch failed: %s", hipGetErrorString(err));
    a.k_new = nullptr;
    a.v_new = nullptr;
  }
  if (opts && opts->event_begin) {
    hipError_t err = hipEventRecord(reinterpret_cast<hipEvent_t>(opts->event_begin), s);
    if (err != hipSuccess) return fail(PA_ERR_HIP, "hipEventRecord(begin) failed: %s", hipGetErrorString(err));
  }
  hipError_t err;
  if (a.casc_width > 0) {
    err = launch_share(a, s);
    if (err != hipSuccess) return fail(PA_ERR_HIP, "shared-prefix detection launch failed: %s", hipGetErrorString(err));
  }
  err = launch_decode(a, dtype, head_dim, p.grid, p.lds, s);
  if (err != hipSuccess) return fail(PA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(err));
  if (opts && opts->event_end) {
    err = hipEventRecord(reinterpret_cast<hipEvent_t>(opts->event_end), s);
    if (err != hipSuccess) return fail(PA_ERR_HIP, "hipEventRecord(end) failed: %s", hipGetErrorString(err));
  }
  if (p.reduce) {
    err = launch_reduce(a, dtype, head_dim, s);
    if (err != hipSuccess) return fail(PA_ERR_HIP, "reduce launch failed: %s", hipGetErrorString(err));
  }
  return ok();
}

}  // namespace

extern "C" {

int pa_paged_attention_decode_ex(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens, float scale, void* out,
                                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                                 int64_t q_seq_stride, int32_t dtype, int32_t out_dtype,
                                 const pa_decode_opts* opts, void* stream) {
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_heads, num_kv_heads,
                     head_dim, block_size, max_blocks_per_seq, num_blocks, q_seq_stride, dtype, out_dtype, opts,
                     stream, nullptr, nullptr, 0, 0);
}

int pa_paged_attention_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                                      void* out, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, int64_t q_seq_stride, int32_t dtype, int32_t out_dtype,
                                      const pa_decode_opts* opts, void* stream) {
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_heads, num_kv_heads,
                     head_dim, block_size, max_blocks_per_seq, num_blocks, q_seq_stride, dtype, out_dtype, opts,
                     stream, nullptr, nullptr, 0, 0, /*noalloc=*/true);
}

int pa_decode_step(const void* q, const void* k_new, const void* v_new, int64_t k_new_stride, int64_t v_new_stride,
                   void* k_cache, void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                   float scale, void* out, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                   int64_t q_seq_stride, int32_t dtype, int32_t out_dtype, const pa_decode_opts* opts,
                   void* stream) {
  if (num_seqs > 0) {
    if (!k_new || !v_new) return fail(PA_ERR_NULL, "k_new and v_new are required");
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (num_kv_heads > 0 && head_dim > 0 && (k_new_stride < row || v_new_stride < row))
      return fail(PA_ERR_SHAPE, "k_new/v_new strides smaller than num_kv_heads*head_dim");
    if (valid_dtype(dtype)) {
      const int e = elem_bytes(dtype);
      if (!aligned16(k_new) || !aligned16(v_new) || (k_new_stride * e) % 16 != 0 || (v_new_stride * e) % 16 != 0)
        return fail(PA_ERR_UNSUPPORTED, "k_new and v_new must be 16-byte aligned with 16-byte strides");
    }
  }
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_heads, num_kv_heads,
                     head_dim, block_size, max_blocks_per_seq, num_blocks, q_seq_stride, dtype, out_dtype, opts,
                     stream, k_new, v_new, k_new_stride, v_new_stride);
}

int pa_paged_attention_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t max_blocks_per_seq, int64_t num_blocks, int64_t q_seq_stride, int32_t dtype,
                              int32_t out_dtype, void* stream) {
  return pa_paged_attention_decode_ex(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                                      num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                                      q_seq_stride, dtype, out_dtype, nullptr, stream);
}

const char* pa_last_error(void) { return t_error.c_str(); }

const char* pa_version(void) { return "libpagedattn 0.1.0 gfx950"; }

int pa_shutdown(void) {
  std::lock_guard<std::mutex> lock(g_mutex);
  int rc = PA_OK;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) cur = -1;
  for (int d = 0; d < kMaxDevices; ++d) {
    DeviceState& st = g_devices[d];
    if (!st.ws) continue;
    if (hipSetDevice(d) != hipSuccess || hipFree(st.ws) != hipSuccess) rc = PA_ERR_HIP;
    st.ws = nullptr;
    st.ws_bytes = 0;
  }
  if (cur >= 0) (void)hipSetDevice(cur);
  if (rc != PA_OK) return fail(rc, "hipFree of a workspace failed");
  return ok();
}

}  // extern "C"
