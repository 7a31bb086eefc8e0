/*
 * pagedattn.h - C ABI of libpagedattn: paged-attention decode for AMD Instinct
 * MI355X (gfx950, CDNA4).
 *
 * What the library computes. The miniVLLM documentation (page "miniVLLM",
 * section "What is miniVLLM?") describes a KV cache kept in fixed-size pages
 * and a paged-attention kernel for the decode phase. The hysenlabs review of
 * MinivLLM (section on the prefilling baseline capped at 128 tokens, closing
 * paragraph) describes the decode benchmark's baselines: a per-sequence loop
 * over the paged cache and a batched gather-and-mask version. Both compute, for
 * every sequence s and query head h, single-query softmax attention over the
 * sequence's L_s cached tokens:
 *
 *     z_t    = scale * <q[s,h,:], K_s[t, h / G, :]>          t = 0 .. L_s - 1
 *     out[s,h,:] = sum_t exp(z_t - max z) V_s[t, h / G, :] / sum_t exp(z_t - max z)
 *
 * with G = num_heads / num_kv_heads query heads per KV head (grouped-query
 * attention: query head h reads KV head h / G). Token t of sequence s lives at
 * offset t % block_size of physical block block_tables[s * max_blocks_per_seq
 * + t / block_size]. The scatter entry point writes each decode step's new
 * K/V rows into cache slots ("KV cache management" in the same section).
 *
 * ----------------------------------------------------------------------------
 * Physical cache layout (fixed by this library, chosen for gfx950 loads)
 *
 *   e = sizeof(element): 4 (fp32) or 2 (fp16, bf16); x = 16 / e.
 *   k_cache: [num_blocks][num_kv_heads][head_dim / x][block_size][x]
 *            key element (block b, head g, offset o, dim d) at
 *            [b][g][d / x][o][d % x]
 *   v_cache: [num_blocks][num_kv_heads][block_size / 4][head_dim][4]
 *            value element (b, g, o, d) at [b][g][o / 4][d][o % 4]
 *
 * Each (block, kv head) page is one contiguous run of block_size * head_dim * e
 * bytes in both caches. Inside it, a 16-byte load of the K page holds 16 bytes
 * of one token's key row, and a load of the V page holds four consecutive
 * tokens of one or two value dims. Those are the operand shapes of the
 * matrix-core instructions the decode kernel uses.
 *
 * ----------------------------------------------------------------------------
 * Conventions for every entry point
 *
 *  - All data pointers are DEVICE pointers on the current HIP device. Scalars
 *    and option structs are host values. `stream` is a hipStream_t passed as
 *    void* (NULL = the default stream).
 *  - Work is enqueued on `stream` and the call returns without synchronising.
 *    The library performs no device-to-host reads, so the calls may be
 *    recorded into a HIP graph once any workspace exists.
 *  - The caller owns every buffer. The library keeps no pointer after a call
 *    except its own workspace.
 *  - Return value: PA_OK (0) on success, otherwise a pa_status code. A thread
 *    local message is available from pa_last_error(). Argument errors are
 *    detected on the host before anything is enqueued.
 *  - Device-side robustness: slots, block ids and context lengths are clamped
 *    or skipped so that no input value causes an access outside the buffers
 *    whose sizes the call describes (see each entry point). Out-of-range values
 *    give unspecified output for the affected sequence, never a fault.
 */
#ifndef PAGEDATTN_H_
#define PAGEDATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_DTYPE = 2,       /* unknown dtype, or inputs of different dtypes */
  PA_ERR_SHAPE = 3,       /* a size is negative/zero where it must be positive, or sizes disagree */
  PA_ERR_UNSUPPORTED = 4, /* valid request outside what the kernels implement (e.g. head_dim 96) */
  PA_ERR_WORKSPACE = 5,   /* caller-provided workspace too small or misaligned */
  PA_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed */
  PA_ERR_CAPACITY = 7     /* not enough free KV blocks (block manager) */
} pa_status;

typedef enum pa_dtype {
  PA_DTYPE_F32 = 0,
  PA_DTYPE_F16 = 1,
  PA_DTYPE_BF16 = 2
} pa_dtype;

/*
 * pa_store_kvcache - write new K/V rows into their cache slots.
 *
 * Passage: miniVLLM documentation, "What is miniVLLM?" (paged KV cache
 * management); hysenlabs MinivLLM review, section on what main.py does (the
 * engine's block allocation and KV cache management during decode).
 *
 * For every token i < num_tokens with slot n = slot_mapping[i] in
 * [0, num_blocks * block_size): for all kv heads g and dims d,
 *     K(block n / block_size, g, offset n % block_size, d) = k[i, g, d]
 *     V(... same ...)                                      = v[i, g, d]
 * as raw bit copies (no conversion; NaN payloads are preserved).
 * Tokens whose slot is negative or >= num_blocks * block_size are skipped.
 * Two tokens with the same slot race (undefined which one lands).
 *
 *   k, v            [num_tokens][num_kv_heads][head_dim] of `dtype`; the two
 *                   inner dims are contiguous; consecutive tokens are
 *                   k_token_stride / v_token_stride ELEMENTS apart
 *                   (>= num_kv_heads * head_dim).
 *   slot_mapping    [num_tokens] int32.
 *   k_cache, v_cache caches in the layout above, num_blocks blocks, `dtype`.
 *   head_dim        multiple of x (16-byte chunks), at most 1024.
 *   block_size      multiple of 4.
 * num_tokens == 0 is a no-op returning PA_OK.
 */
int pa_store_kvcache(const void* k, const void* v, const int32_t* slot_mapping,
                     void* k_cache, void* v_cache,
                     int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int64_t num_blocks,
                     int64_t k_token_stride, int64_t v_token_stride,
                     int32_t dtype, void* stream);

/*
 * pa_paged_attention_decode - single-query attention through block tables.
 *
 * Passage: miniVLLM documentation, "What is miniVLLM?" (paged attention for
 * decode) and "Explore by topic" (online softmax); hysenlabs MinivLLM review,
 * section on the prefilling baseline capped at 128 tokens (the decode
 * benchmark's loop and gather-and-mask baselines compute the same result).
 * The formula is in the file header.
 *
 *   q             [num_seqs][num_heads][head_dim] of `dtype`; heads and dims
 *                 contiguous, consecutive sequences q_seq_stride ELEMENTS apart
 *                 (>= num_heads * head_dim).
 *   k_cache, v_cache  num_blocks blocks in the layout above, `dtype`.
 *   block_tables  [num_seqs][max_blocks_per_seq] int32, contiguous; the whole
 *                 table must be readable. Entries past ceil(L_s / block_size)
 *                 never affect the result (the kernel may read them to warm
 *                 its cache, but never uses their values). An entry outside
 *                 [0, num_blocks) is clamped into range (unspecified output).
 *   context_lens  [num_seqs] int32, L_s. Values are clamped to
 *                 [0, max_blocks_per_seq * block_size]. L_s == 0 gives zeros.
 *   scale         softmax scale, applied in fp32 (usually 1/sqrt(head_dim)).
 *   out           [num_seqs][num_heads][head_dim], contiguous, of out_dtype:
 *                 PA_DTYPE_F32, or the same dtype as q (rounded to nearest even
 *                 from the fp32 result).
 *   Supported: dtype fp32/fp16/bf16; head_dim 64, 128 or 256; block_size a
 *   power of two in [16, 256]; num_heads a multiple of num_kv_heads (any
 *   group size G; groups above 16 heads are processed 16 at a time).
 *   num_seqs at most 16383.
 *
 * Long contexts are split across wavefronts and the pieces are merged by a
 * second kernel (log-sum-exp weighting); see pa_decode_opts. Uses a workspace
 * owned by the library, allocated or grown on first use for a given size
 * (that call is not graph-capturable; later calls of the same or smaller size
 * are). pa_shutdown() frees it. Calls on one device share that workspace, so
 * calls that may overlap (different streams) must use pa_paged_attention_decode_ex
 * with workspaces of their own.
 */
int pa_paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              float scale, void* out,
                              int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              int64_t num_blocks, int64_t q_seq_stride,
                              int32_t dtype, int32_t out_dtype, void* stream);

/*
 * Options for pa_paged_attention_decode_ex.
 *
 * partition_size (tokens):
 *    0  automatic: when no context can exceed 512 tokens
 *       (max_blocks_per_seq * block_size <= 512), the workgroup split (-3) if
 *       every (sequence, kv head, head group) context gets a resident
 *       workgroup of its own (at most 2 * compute units of them), else one
 *       pass (-1); balanced ranges (-2) otherwise. Decided on the host from
 *       the sizes alone.
 *   -1  one pass: every (sequence, kv head) context is handled whole by one
 *       wavefront; no reduce kernel runs.
 *   -2  balanced ranges: the concatenated 16-token tiles of all (sequence,
 *       kv head) contexts are divided evenly over the wavefronts the device
 *       holds at once, so long and short sequences finish together; contexts
 *       cut by a range boundary are merged by the reduce kernel.
 *   -3  workgroup split: each (sequence, kv head) context is handled by one
 *       workgroup, whose four wavefronts stream equal shares of its tiles at
 *       once and merge their partial results in LDS (same log-sum-exp merge as
 *       the reduce kernel); no workspace and no reduce kernel. Shortens the
 *       per-context chain of small batches. Where the four partial rows would
 *       exceed 64 KiB of LDS (head_dim 256 with 16 query heads per kv head) it
 *       runs as one pass.
 *   >0  fixed ranges of partition_size tokens (a multiple of 16) over the same
 *       concatenated tile stream. The device's resident wavefronts loop over
 *       the ranges; the workspace has rows for the ranges of the longest
 *       possible batch (every context max_blocks_per_seq * block_size long).
 * cached_prefix_tokens: K/V of the first cached_prefix_tokens tokens of every
 *       context are read with the default cache policy; later tokens are read
 *       with the non-temporal (streaming) policy, which moves single-use data
 *       faster but does not keep it in the last-level cache. Prefix caching
 *       shares the leading blocks of contexts between sequences, so those are
 *       the reads worth keeping. 0 = library default
 *       (PA_DEFAULT_CACHED_PREFIX_TOKENS), -1 = stream everything, INT32_MAX =
 *       never stream. Changes speed only, never results.
 * workspace / workspace_bytes: device memory used instead of the library's own
 *       (NULL = library-owned). Must be 256-byte aligned and at least
 *       pa_decode_workspace_bytes(...) bytes (pa_decode_plan_ex's figure with
 *       shared_prefix). Its contents need no initialisation. Calls that share
 *       a workspace must not overlap.
 * event_begin / event_end: optional hipEvent_t handles (as void*) recorded on
 *       `stream` immediately before and after the attention kernel itself (not
 *       the reduce kernel), so callers can time that kernel alone. With
 *       shared_prefix they also enclose the detection kernel.
 * shared_prefix: nonzero = read shared prefixes once. Prefix caching (miniVLLM
 *       docs, "What is miniVLLM?") lets sequences share the physical blocks of
 *       a common prefix. With this option a first small kernel finds, in each
 *       window of W = 16 / G consecutive sequences, the group whose leading
 *       block-table entries are identical (equal physical ids, so equal K/V),
 *       and the prefix length that saves the most reads. It counts only whole
 *       blocks before each sequence's last-token block, and groups need a
 *       prefix of two 16-token tiles or more. The attention kernel then streams
 *       the group's prefix once, the G query heads of the group's sequences
 *       filling the 16 columns of one matrix-core tile. Each sequence streams
 *       its own remaining tiles, and the reduce kernel merges its partials with
 *       the prefix's (the same log-sum-exp merge). The result is the same
 *       attention (a different summation order). Sharing is verified on the device
 *       from the block tables, so the option is a hint that costs time when
 *       nothing is shared and never changes what is computed. Applies only in
 *       the split modes (-2 or a fixed size; with the automatic mode, where it
 *       picks them), with G <= 8 and num_seqs <= 8191; otherwise ignored. The
 *       workspace grows: see pa_decode_plan_ex.
 */
#define PA_DEFAULT_CACHED_PREFIX_TOKENS 1024

typedef struct pa_decode_opts {
  int32_t partition_size;
  int32_t cached_prefix_tokens;
  void* workspace;
  size_t workspace_bytes;
  void* event_begin;
  void* event_end;
  int32_t shared_prefix;
} pa_decode_opts;

int pa_paged_attention_decode_ex(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 float scale, void* out,
                                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                 int64_t num_blocks, int64_t q_seq_stride,
                                 int32_t dtype, int32_t out_dtype,
                                 const pa_decode_opts* opts, void* stream);

/*
 * pa_paged_attention_decode_noalloc - pa_paged_attention_decode_ex without any
 * device-memory allocation.
 *
 * For callers that cannot allocate: code being recorded into a HIP graph,
 * serving loops that must not call the allocator, harnesses that forbid it.
 * Arguments, result and errors as for pa_paged_attention_decode_ex (the same
 * kernels run), except:
 *  - The split modes' workspace is a fixed array of PA_NOALLOC_SCRATCH_BYTES
 *    of device memory inside the library, one per device, held from the first
 *    call on that device until the process ends. That first call looks up the
 *    array's device address (set-up, outside any graph capture); no call
 *    allocates, frees or calls an allocating routine.
 *  - opts->workspace must be NULL (PA_ERR_WORKSPACE otherwise).
 *  - A call whose plan needs more workspace than PA_NOALLOC_SCRATCH_BYTES
 *    (pa_decode_plan_ex reports the figure) returns PA_ERR_WORKSPACE and
 *    enqueues nothing. One pass and workgroup split need none.
 *  - Every call on a device uses that device's one array, which keeps the last
 *    call's contents (nothing in it needs to start at zero). Calls that may
 *    overlap on one device (other streams, other host threads) race on it: the
 *    caller must serialise them.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)

int pa_paged_attention_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      float scale, void* out,
                                      int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, int64_t q_seq_stride,
                                      int32_t dtype, int32_t out_dtype,
                                      const pa_decode_opts* opts, void* stream);

/*
 * pa_decode_step - the decode step's scatter and attention in one launch.
 *
 * Same result as pa_store_kvcache of each sequence's new token followed by
 * pa_paged_attention_decode_ex: for every sequence s with L_s = context_lens[s]
 * >= 1, the token at position L_s - 1 (offset (L_s-1) % block_size of block
 * block_tables[s][(L_s-1) / block_size]) gets k_new[s] / v_new[s] in the
 * caches (bit copies), and the attention over tokens 0 .. L_s-1 uses them.
 * The wavefront that computes the tile holding that token takes the new K/V
 * from k_new/v_new directly and writes them to the cache slot, so no separate
 * scatter kernel runs. Passage: as for the two entry points it fuses (the
 * decode step of the paged engine, miniVLLM docs, "What is miniVLLM?").
 *
 *   k_new, v_new  [num_seqs][num_kv_heads][head_dim] of `dtype`, inner dims
 *                 contiguous, sequences k_new_stride / v_new_stride ELEMENTS
 *                 apart; 16-byte aligned rows.
 *   Other arguments as for pa_paged_attention_decode_ex (k_cache/v_cache are
 *   written). Each new token's slot must not hold another token of the same
 *   step (slot uniqueness, as for pa_store_kvcache).
 */
int pa_decode_step(const void* q, const void* k_new, const void* v_new, int64_t k_new_stride, int64_t v_new_stride,
                   void* k_cache, void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                   float scale, void* out, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                   int64_t q_seq_stride, int32_t dtype, int32_t out_dtype, const pa_decode_opts* opts,
                   void* stream);

/*
 * pa_paged_prefill - causal attention of each sequence's new tokens over its
 * paged KV cache (flash-attention prefill with online softmax: miniVLLM docs,
 * "What is miniVLLM?" and "Explore by topic"; the materialised standard form
 * is in the hysenlabs MinivLLM review, prefilling-baseline section).
 *
 * Sequence s owns query rows query_start[s] .. query_start[s+1]-1 of q; with
 * n_s of them and L_s = context_lens[s] cached tokens (the new tokens' K/V
 * already stored, e.g. with pa_store_kvcache), query i sits at position
 * L_s - n_s + i and attends to tokens 0 .. L_s - n_s + i. n_s = L_s is a full
 * prefill, n_s < L_s continues after cached tokens (prefix-cache hit, chunked
 * prefill), n_s = 1 is a decode step. Rows of q past L_s new tokens, or of a
 * sequence with L_s = 0, are left unwritten in out.
 *
 *   q            [num_tokens][num_heads][head_dim], heads and dims contiguous,
 *                tokens q_token_stride ELEMENTS apart.
 *   query_start  [num_seqs + 1] int32, non-decreasing, query_start[num_seqs]
 *                <= num_tokens. Being device memory it is not checked: values
 *                are clamped into [0, num_tokens] (and each sequence's end to
 *                at least its start), so malformed content gives meaningless
 *                rows but never a q read or out write outside the buffers.
 *   out          [num_tokens][num_heads][head_dim] contiguous, fp32 or dtype.
 *   Other arguments and limits as for pa_paged_attention_decode.
 * Workgroups take their work items from counters in a small fixed array of the library (no
 * allocation; every launch leaves its counters at zero when it ends, so calls can be recorded
 * into a HIP graph). Calls take the 1024 sets of counters in turn: calls that run at the same time
 * on one device (other streams, other host threads) must not number 1024 or more, or two of them
 * may share counters and skip work. A captured call keeps the set it took at capture. Replays of
 * one executable graph are ordered and never overlap, but two executable graphs instantiated
 * from one capture share that set: the caller must not run them at the same time.
 */
int pa_paged_prefill(const void* q, int64_t q_token_stride, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                     float scale, void* out, int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                     int64_t num_blocks, int32_t dtype, int32_t out_dtype, void* stream);

/*
 * Launch plan of a decode call: pure host arithmetic, no device access when
 * num_cus > 0 (num_cus <= 0 queries the current device). Fills any non-NULL
 * output: the wavefront count of the attention kernel; range_tokens, the
 * tokens per wavefront range (> 0 fixed, 0 balanced over the data, -1 one
 * pass, -3 workgroup split); whether the reduce kernel runs; and the workspace bytes the call
 * needs. Returns the pa_status the decode call would return for these sizes.
 */
int pa_decode_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t max_blocks_per_seq, int32_t dtype,
                   int32_t partition_size, int32_t num_cus,
                   int64_t* num_waves, int32_t* range_tokens, int32_t* uses_reduce,
                   size_t* workspace_bytes);

/*
 * pa_decode_plan_ex - the same plan for a call with these options (partition_size
 * and shared_prefix are read; opts may be NULL). Also fills shared_prefix_window:
 * the sequences per shared-prefix window, 0 when shared prefixes do not apply.
 */
int pa_decode_plan_ex(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t max_blocks_per_seq, int32_t dtype,
                      const pa_decode_opts* opts, int32_t num_cus,
                      int64_t* num_waves, int32_t* range_tokens, int32_t* uses_reduce,
                      int32_t* shared_prefix_window, size_t* workspace_bytes);

/* Workspace bytes pa_paged_attention_decode_ex needs for these sizes without shared_prefix
 * (0 on bad arguments). */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                 int32_t dtype, int32_t partition_size);

/*
 * pa_copy_blocks - copy whole KV blocks (both caches, all kv heads): for each
 * i < num_pairs, block dst[i] becomes a bit copy of block src[i]. Used for the
 * block manager's copy-on-write. src/dst are DEVICE int32 arrays; pairs with an
 * id outside [0, num_blocks) are skipped; a dst equal to another pair's src or
 * dst races. Layout and dtype as for pa_store_kvcache.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst, int32_t num_pairs,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                   int32_t dtype, void* stream);

/* ----------------------------------------------------------------------------
 * Block manager (host memory only, no device work): the allocator that turns
 * sequences of token ids into block tables and slot mappings, with prefix
 * caching. Passage: miniVLLM docs, "What is miniVLLM?" (paged KV cache with
 * prefix caching); hysenlabs MinivLLM review, "The structure block ..." (block
 * management for the KV cache) and its dependency list (token hashing).
 *
 * Full blocks are keyed by a chained 64-bit hash of all tokens up to and
 * including them; a new sequence reuses every leading full block whose key and
 * token ids match a cached block (reference counted). Freed full blocks stay
 * cached until evicted (least recently freed first) when free blocks run out.
 * Block ids are in [0, num_blocks); slot = block * block_size + offset.
 * All functions are thread-safe per manager; errors return a pa_status with a
 * message from pa_bm_last_error().
 */
typedef struct pa_block_manager pa_block_manager;

/* New manager over num_blocks blocks of block_size tokens; NULL on bad sizes. */
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager* m);

/* Registers a sequence with its prompt tokens and allocates its blocks. On
 * success *num_cached_tokens (if non-NULL) is the number of leading tokens whose
 * blocks were already cached (their K/V need not be recomputed or stored).
 * PA_ERR_CAPACITY if the blocks do not fit (nothing is changed then). */
int pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                       int32_t* num_cached_tokens);

/* Reserves the slot of one new token of a sequence (a decode step). If the
 * sequence's last block was shared and partially filled, a fresh block replaces
 * it and *copy_src / *copy_dst name the block copy the caller must perform on
 * the device before storing the token (both -1 otherwise). */
int pa_bm_append_token(pa_block_manager* m, int64_t seq_id, int32_t token, int32_t* slot, int32_t* copy_src,
                       int32_t* copy_dst);

/* New sequence child_id sharing all blocks of parent_id (parallel sampling). */
int pa_bm_fork(pa_block_manager* m, int64_t parent_id, int64_t child_id);

/* Releases a sequence's blocks. */
int pa_bm_free_sequence(pa_block_manager* m, int64_t seq_id);

/* Copies the sequence's block ids into out[0 .. n) (n <= max_blocks) and
 * reports n and the token count; out may be NULL to query sizes only. */
int pa_bm_block_table(pa_block_manager* m, int64_t seq_id, int32_t* out, int32_t max_blocks, int32_t* num_blocks,
                      int32_t* num_tokens);

/* Slots of tokens [first_token, first_token + count) of a sequence. */
int pa_bm_slots(pa_block_manager* m, int64_t seq_id, int32_t first_token, int32_t count, int32_t* slots);

/* Free-or-evictable blocks, cached (hashed) blocks, and hit/miss/eviction counters. */
int pa_bm_stats(pa_block_manager* m, int32_t* free_blocks, int32_t* cached_blocks, int64_t* hits, int64_t* misses,
                int64_t* evictions);

/* Reference count of a block (-1 for a bad id). */
int32_t pa_bm_block_ref(pa_block_manager* m, int32_t block);

/* Message of the last failed block-manager call on this thread ("" if none). */
const char* pa_bm_last_error(void);

/* Message of the last failed call on this thread ("" if none). Never NULL. */
const char* pa_last_error(void);

/* Library version string, e.g. "libpagedattn 0.1.0 gfx950". */
const char* pa_version(void);

/*
 * Frees the library-owned workspaces of all devices. hipFree waits for the
 * device's queued work first, so kernels already launched finish with their
 * workspace; no decode call may run concurrently with this one. A later decode
 * call allocates a workspace again. Returns PA_OK or PA_ERR_HIP.
 */
int pa_shutdown(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H_ */
