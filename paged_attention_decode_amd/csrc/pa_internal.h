// Internal declarations shared by the libpagedattn translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

inline int elem_bytes(int dt) { return dt == kF32 ? 4 : 2; }

// Tokens per matrix-core tile: one 16x16 output tile covers 16 tokens.
constexpr int kTile = 16;
// Threads per workgroup of the attention kernel (four wave64 wavefronts).
constexpr int kDecodeThreads = 256;
constexpr int kWavesPerGroup = kDecodeThreads / 64;
// Query heads handled together by one wavefront (columns of a 16x16 tile).
constexpr int kHeadsPerTile = 16;
// Largest batch: per-sequence tile prefix sums live in LDS (4 bytes each).
constexpr int kMaxSeqs = 16383;
// Largest batch for shared-prefix decode: the per-sequence sharing words also live in LDS.
constexpr int kMaxSharedSeqs = 8191;
// Split modes: LDS a workgroup may use for the prefix sums plus the deferred-row slots, and the
// most slots per wavefront.
constexpr int kStashLdsBytes = 65536;
constexpr int kMaxStashSlots = 8;
// Shared-prefix word of a sequence (0: the sequence reads its whole context itself):
// bits 0-15 the prefix length in 16-token tiles, bits 16-19 the window slot of the group's
// leader (whose block table the prefix is read through), bit 20 set.
constexpr int kShareIncluded = 1 << 20;
__host__ __device__ inline int share_tiles(int w) { return w & 0xFFFF; }
__host__ __device__ inline int share_leader(int w) { return (w >> 16) & 15; }
// partition_size (and DecodeArgs::range_tiles) of the workgroup-split mode: the wavefronts of a
// workgroup share one segment's tiles and merge their partial results in LDS.
constexpr int kWorkgroupSplit = -3;
// Balanced mode never gives a wavefront fewer tiles than this.
#ifndef PA_MIN_TILES_PER_WAVE
#define PA_MIN_TILES_PER_WAVE 2
#endif
constexpr int kMinTilesPerWave = PA_MIN_TILES_PER_WAVE;

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  // Normalised partial outputs, one row of head_dim floats each, and their log2-sum-exp2:
  // rows [ranges][2][ws_cols] for pieces cut by range boundaries, then (shared prefixes only)
  // whole_own_row.. [num_seqs * segs_per_seq][gh_max] and whole_pre_row..
  // [windows * segs_per_seq][16] for whole segments that are still merged.
  float* ws_o;
  float* ws_lse;
  int64_t whole_own_row;
  int64_t whole_pre_row;
  int4* ws_meta;      // [num_seqs * segs_per_seq] {first range, its slot, last range, 0}
  // Shared prefixes (casc_width > 0): per-sequence words written by the detection kernel, and
  // the pieces of each window's prefix segments, [ceil(num_seqs / casc_width) * segs_per_seq].
  int32_t* ws_share;
  int4* ws_meta_pre;
  int64_t q_seq_stride;   // elements
  int64_t num_blocks;
  float scale_log2;       // scale * log2(e)
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;          // query heads per kv head
  int32_t n_hg;           // ceil(group / 16): head groups per kv head
  int32_t gh_max;         // min(group, 16)
  int32_t segs_per_seq;   // num_kv_heads * n_hg
  int32_t block_size;
  int32_t bs_log2;
  int32_t max_blocks;     // block table row length
  int32_t out_f32;        // 1: fp32 output, 0: output in the input dtype
  int32_t num_waves;      // wavefronts launched
  int32_t range_tiles;    // >0 fixed tiles per wavefront, 0 balanced, -1 one pass, kWorkgroupSplit
  int32_t cached_prefix_tokens;  // tiles starting before this token use cached loads, later ones stream
  int32_t ws_cols;        // partial-output columns per (range, slot): gh_max, or 16 with shared prefixes
  int32_t casc_width;     // sequences per shared-prefix window (16 / group), 0 = no prefix sharing
  // Split modes: LDS slots per wavefront that hold finished rows until its last tile is done
  // (0: rows are written at once), their size in floats, and where the slots start (floats from
  // the start of the dynamic LDS).
  int32_t stash_slots;
  int32_t stash_slot_floats;
  int32_t stash_off;
  // Fused scatter of the step's token at position L-1 (null: plain decode).
  const void* k_new;      // [num_seqs][num_kv_heads][head_dim]
  const void* v_new;
  int64_t k_new_stride;   // elements between sequences
  int64_t v_new_stride;
};

struct StoreArgs {
  const void* k;
  const void* v;
  const int32_t* slot_mapping;
  void* k_cache;
  void* v_cache;
  int64_t k_stride;   // elements between tokens
  int64_t v_stride;
  int64_t num_slots;  // num_blocks * block_size
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
};

// Sets of prefill work-queue counters; the host hands them to calls in turn.
constexpr int kQueueSlots = 1024;

struct PrefillArgs {
  const void* q;                // [num_tokens][num_heads][head_dim], token stride q_token_stride
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;   // [num_seqs + 1]
  void* out;                    // [num_tokens][num_heads][head_dim]
  int64_t q_token_stride;
  int64_t num_blocks;
  float scale_log2;
  int32_t num_seqs;
  int32_t num_tokens;           // rows of q and out
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t n_hg;
  int32_t gh_max;
  int32_t block_size;
  int32_t bs_log2;
  int32_t max_blocks;
  int32_t out_f32;
  int32_t num_waves;
  int32_t queue_slot;           // which set of work-queue counters this call uses (< kQueueSlots)
};

// Launchers (return the launch error, hipSuccess otherwise).
hipError_t launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int grid, size_t lds_bytes,
                          hipStream_t stream);
// Query tokens one prefill work item covers (per wavefront; a shared-variant workgroup covers
// kWavesPerGroup times as many).
int prefill_queries_per_item(int dtype, int head_dim, int gh_max);
// Workgroup-shared prefill (16-bit inputs, head_dim 128): its two LDS step buffers.
size_t prefill_shared_buffer_bytes(int head_dim);
hipError_t launch_prefill_shared(const PrefillArgs& a, int dtype, int head_dim, int grid, size_t lds_bytes,
                                 hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int grid, size_t lds_bytes,
                         hipStream_t stream);
hipError_t launch_reduce(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream);
// Fused decode step: whether the attention kernel takes the step's token itself; where it does
// not, launch_append writes the token of every (sequence, kv head) to its cache slot first.
bool decode_fuses_step(int dtype, int head_dim);
hipError_t launch_append(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream);
// Shared-prefix detection: fills a.ws_share (one workgroup per window of a.casc_width sequences).
hipError_t launch_share(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_store(const StoreArgs& a, int dtype, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst,
                              int32_t num_pairs, int64_t block_bytes, int64_t num_blocks, hipStream_t stream);
// Resident workgroups of the attention kernel per compute unit for this LDS size.
hipError_t decode_groups_per_cu(int dtype, int head_dim, size_t lds_bytes, int* groups);

}  // namespace pa
