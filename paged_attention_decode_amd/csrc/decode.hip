// Paged-attention decode kernels for gfx950 (CDNA4).
//
// Operation: single-query softmax attention of every (sequence, query head)
// over the sequence's cached tokens, read through its block table
// (miniVLLM documentation, "What is miniVLLM?": paged attention for decode
// over a paged KV cache; online softmax as in "Explore by topic" there and in
// the tiny-vllm note, "Chi tiết"). The formula is in include/pagedattn.h.
//
// Work decomposition. A segment is one (sequence, kv head, group of up to 16
// query heads); it has ceil(L/16) tiles of 16 tokens. The tiles of all
// segments are concatenated in (sequence, kv head, head group) order and cut
// into equal ranges, one per wavefront, so every wavefront streams the same
// number of KV bytes however skewed the lengths are. A segment that lies
// inside one range is finished by its wavefront (output written directly);
// a segment cut by range boundaries leaves one normalised partial output and
// its log2-sum-exp2 per piece, merged afterwards by reduce_kernel. A wavefront
// keeps the rows it finishes in LDS and writes them after its last tile: on
// gfx9-family GPUs a store shares the wait counter of the loads, and waiting
// for its acknowledgement behind a full read stream would stall the next tiles.
//
// Shared prefixes (an option; prefix caching shares the physical blocks of a
// common prefix between sequences): share_kernel finds, per window of 16/G
// sequences, a group whose leading block-table entries are the same blocks.
// The group's prefix then forms segments of its own, whose 16 columns are the
// group members' heads, read once; each member's own segments start after it,
// and the merge combines both.
//
// Per 16-token tile, one wavefront computes
//   S[t][h]   = K[t][:] . Q[h][:]          (matrix core: rows = tokens, cols = heads)
//   online softmax on S (running max m, running sum l, per head = per lane column)
//   O^T[d][h] += V^T[d][t] . P^T[t][h]     (matrix core: rows = dims, cols = heads)
// The result layout of the first product (lane = 16*row_group + head, four
// token rows per lane) is exactly the operand layout the second product needs
// for P^T, so P never leaves registers. The cache layout (pagedattn.h) makes
// every 16-byte global load land directly in the operand registers of these
// instructions: no LDS staging, no transposes. K/V of the next tile are in
// flight while the current tile is computed.
//
// Numerics: products and accumulation in fp32. For fp16/bf16 inputs the
// softmax weights P enter the second product as a sum of two 16-bit numbers
// (rounded value + rounded remainder), so the weights keep ~16 significant
// bits instead of 8 (bf16) or 11 (fp16).

#include "device_common.h"

#include <type_traits>

namespace pa {
namespace {

using namespace dev;

template <int DT, int D, bool FUSE>
struct Piece {
  using C = Cfg<DT, D>;

  // Runs tiles [lt0, lt1) of segment (s, r). complete: the piece is the whole
  // segment, so the normalised result goes straight to `out`; otherwise to
  // part_o / part_lse (rows of the group's heads, in LDS) when given, else to
  // workspace rows row_base + column.
  // cols != 0: a shared prefix. The tiles are read through sequence s's block table, and the
  // columns are the kv head's query heads of the sequences win + m for each bit m of cols
  // (column m * group + head); the result always goes to the workspace, all 16 columns.
  // stash != null: the rows are not written here but left in that LDS slot (header words 0-5,
  // values from float 16, lse values after the rows), and write_stashed writes them later.
  static __device__ __forceinline__ void run(const DecodeArgs& a, int s, int r, int L, int lt0, int lt1,
                                             bool complete, int64_t row_base, int lane,
                                             float* part_o = nullptr, float* part_lse = nullptr,
                                             int win = 0, int cols = 0, float* stash = nullptr) {
    // All of these are the same in every lane. Saying so lets the compiler keep what derives
    // from them in scalar registers, and read the block table with scalar loads.
    s = __builtin_amdgcn_readfirstlane(s);
    r = __builtin_amdgcn_readfirstlane(r);
    L = __builtin_amdgcn_readfirstlane(L);
    lt0 = __builtin_amdgcn_readfirstlane(lt0);
    lt1 = __builtin_amdgcn_readfirstlane(lt1);
    win = __builtin_amdgcn_readfirstlane(win);
    cols = __builtin_amdgcn_readfirstlane(cols);
    const int kq = lane >> 4;  // operand k-group, and result row group
    const int ln = lane & 15;  // operand row, and result column (= head in group)
    const int g = r / a.n_hg;
    const int hg = r - g * a.n_hg;
    const int h0 = g * a.group + hg * kHeadsPerTile;
    const int gh = min(kHeadsPerTile, a.group - hg * kHeadsPerTile);
    const int bs = a.block_size;
    const bool shared = cols != 0;

    // Query operand: row of column ln, 16-byte chunk 4j + kq. The resource covers the column
    // rows only, and a padding column's offset lies past its end, so padding columns read zeros
    // with no branch around the loads.
    bool valid;
    u4 qv[C::kLoads];
    {
      const char* qg;
      int qbytes, qoff;
      if (shared) {
        const int m = ln / a.group;
        const int hl = ln - m * a.group;
        valid = ((cols >> m) & 1) != 0;
        const int rows = min(a.casc_width, a.num_seqs - win);
        qg = reinterpret_cast<const char*>(a.q) + ((int64_t)win * a.q_seq_stride + (int64_t)g * a.group * D) * C::kE;
        qbytes = (int)(((int64_t)(rows - 1) * a.q_seq_stride + (int64_t)a.group * D) * C::kE);
        qoff = valid ? (int)(((int64_t)m * a.q_seq_stride + (int64_t)hl * D) * C::kE) : qbytes;
      } else {
        valid = ln < gh;
        qg = reinterpret_cast<const char*>(a.q) + ((int64_t)s * a.q_seq_stride + (int64_t)h0 * D) * C::kE;
        qbytes = gh * D * C::kE;
        qoff = ln * D * C::kE;
      }
      const __amdgpu_buffer_rsrc_t qr = page_rsrc(qg, qbytes);
#pragma unroll
      for (int j = 0; j < C::kLoads; ++j) qv[j] = buf_load16<kPolicyDefault>(qr, qoff + (4 * j + kq) * 16);
    }

    f4 acc[C::kAcc];
#pragma unroll
    for (int u = 0; u < C::kAcc; ++u) acc[u] = f4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;
    float l = 0.f;

    if (L > 0) {
      const int64_t page_bytes = (int64_t)bs * D * C::kE;
      const int page_bytes32 = (int)page_bytes;
      const int64_t blk_stride = (int64_t)a.num_kv_heads * page_bytes;
      const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (int64_t)g * page_bytes;
      const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (int64_t)g * page_bytes;
      const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;
      const int64_t nb_max = a.num_blocks - 1;
      // Lane offsets inside a page. K: chunk (4j + kq) of token (off0 + ln).
      // V (16-bit): dims 32w + 2ln, +1 of tokens off0 + 4kq .. +3.
      // V (fp32):   dim 16u + ln of tokens off0 + 4kq .. +3.
      const uint32_t k_lane = (uint32_t)((kq * bs + ln) * 16);
      const uint32_t v_lane = (DT == kF32) ? (uint32_t)((kq * D + ln) * 16) : (uint32_t)((kq * D + 2 * ln) * 8);

      // Block-table entries come from scalar loads (their own wait counter), one tile ahead.
      // Tiles past the piece read the piece's last page entry and load nothing (below).
      const_i32* cbt = (const_i32*)bt;
      const int last_page = ((lt1 - 1) * kTile) >> a.bs_log2;
      auto bt_entry = [&](int i) -> int { return cbt[min((i * kTile) >> a.bs_log2, last_page)]; };

      // Fused scatter (pa_decode_step): the step's new token sits at position L-1, in
      // row r0 of tile tl. The wavefront computing that tile takes its K/V from
      // k_new/v_new (patched into the loaded registers) and, for head group 0,
      // writes them to the token's cache slot.
      const int tl = (L - 1) >> 4;
      const int r0 = (L - 1) & (kTile - 1);
      const bool fuse = FUSE && !shared && tl >= lt0 && tl < lt1;
      u4 knew[C::kLoads];           // key chunk 4j + kq (used by the lanes of row r0)
      uint32_t vnew[C::kLoads];     // value dims 32w + 2ln, +1 (16-bit) or dim 16u + ln (fp32)
      int64_t blk_new = 0;
      if (fuse) {
        // Loaded before the tile loop: older than every tile load, so they add no waits inside it.
        const char* kn = reinterpret_cast<const char*>(a.k_new) + ((int64_t)s * a.k_new_stride + (int64_t)g * D) * C::kE;
        const char* vn = reinterpret_cast<const char*>(a.v_new) + ((int64_t)s * a.v_new_stride + (int64_t)g * D) * C::kE;
#pragma unroll
        for (int j = 0; j < C::kLoads; ++j) {
          knew[j] = *reinterpret_cast<const u4*>(kn + (4 * j + kq) * 16);
          vnew[j] = (DT == kF32) ? *reinterpret_cast<const uint32_t*>(vn + (16 * j + ln) * 4)
                                 : *reinterpret_cast<const uint32_t*>(vn + (32 * j + 2 * ln) * 2);
        }
      }

      // Issues tile i's K/V loads with cache policy POL; raw = its page's block-table entry;
      // t_hi = end of the tiles being streamed. Every loop position issues the same loads, so
      // the compiler's wait counts stay exact and the next tile's loads stay in flight while
      // this one is computed.
      auto load_tile = [&](auto pol, int i, int raw, int t_hi, u4 (&kb)[C::kLoads], u4 (&vb)[C::kLoads]) {
        constexpr int POL = decltype(pol)::value;
        const int t0 = i * kTile;
        const int off0 = t0 & (bs - 1);
        int64_t blk = __builtin_amdgcn_readfirstlane(raw);
        blk = blk < 0 ? 0 : (blk > nb_max ? nb_max : blk);
        if (fuse && i == tl) blk_new = blk;
        // One buffer resource per page: the page's base in scalar registers,
        // 32-bit lane offsets, and loads past the resource's end return zero. A tile past
        // t_hi gets an empty resource: its loads return zeros and read no memory.
        const int bytes = i < t_hi ? page_bytes32 : 0;
        const __amdgpu_buffer_rsrc_t kr = page_rsrc(kbase + blk * blk_stride, bytes);
        const __amdgpu_buffer_rsrc_t vr = page_rsrc(vbase + blk * blk_stride, bytes);
        const int koff = (int)k_lane + off0 * 16;
        const int voff = (int)v_lane + off0 * D * C::kE;
#pragma unroll
        for (int j = 0; j < C::kLoads; ++j) kb[j] = buf_load16<POL>(kr, koff + j * 64 * bs);
#pragma unroll
        for (int j = 0; j < C::kLoads; ++j) vb[j] = buf_load16<POL>(vr, voff + j * 256);
      };

      auto compute_tile = [&](int i, int t_hi, u4 (&kb)[C::kLoads], u4 (&vb)[C::kLoads]) {
        if (fuse && i == tl) {
          const int i0 = r0 & 3;
          const bool krow = ln == r0, vrow = kq == (r0 >> 2);
          const int off0 = (tl * kTile) & (bs - 1);
          char* kdst = const_cast<char*>(kbase) + blk_new * blk_stride + (int64_t)k_lane + off0 * 16;
          char* vdst = const_cast<char*>(vbase) + blk_new * blk_stride + (int64_t)v_lane + (int64_t)off0 * D * C::kE;
          // With a merge kernel (split modes) that kernel writes the slot, so this one never
          // waits on stores; one pass has no merge kernel and writes here.
          const bool write = hg == 0 && a.range_tiles < 0;
#pragma unroll
          for (int j = 0; j < C::kLoads; ++j) {
            if (krow) {
              kb[j] = knew[j];
              if (write) *reinterpret_cast<u4*>(kdst + j * 64 * bs) = knew[j];
            }
            if (vrow) {
              if constexpr (DT == kF32) {
#pragma unroll
                for (int c = 0; c < 4; ++c) vb[j][c] = (c == i0) ? vnew[j] : vb[j][c];
                if (write) *reinterpret_cast<u4*>(vdst + j * 256) = vb[j];
              } else {
                // dword c holds tokens 2c, 2c+1 of the even dim (c < 2) or of the odd dim (c >= 2)
                const uint32_t lo = vnew[j] & 0xFFFFu, hi = vnew[j] >> 16;
                const uint32_t keep = (i0 & 1) ? 0x0000FFFFu : 0xFFFF0000u;
                const int sh = (i0 & 1) * 16;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                  const uint32_t nv = (c < 2 ? lo : hi) << sh;
                  vb[j][c] = ((c & 1) == (i0 >> 1)) ? ((vb[j][c] & keep) | nv) : vb[j][c];
                }
                // The lane's 16 bytes are four tokens of two dims; writing them back whole stores
                // the new token and returns the other three the bits just loaded (same block,
                // which only this sequence writes).
                if (write) *reinterpret_cast<u4*>(vdst + j * 256) = vb[j];
              }
            }
          }
        }
        // S[token 4kq + r][head ln] for r = 0..3
        f4 sv = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < C::kLoads; ++j) {
          if constexpr (DT == kF32) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sv = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kb[j][e]), __uint_as_float(qv[j][e]), sv, 0, 0, 0);
          } else if constexpr (DT == kBF16) {
            sv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, kb[j]), __builtin_bit_cast(b8, qv[j]), sv, 0, 0, 0);
          } else {
            sv = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, kb[j]), __builtin_bit_cast(h8, qv[j]), sv, 0, 0, 0);
          }
        }
        const int t0 = i * kTile;
        const bool partial = (t0 + kTile > L);
        // past t_hi: a filler tile of the last round, every key masked
        const int t_end = i < t_hi ? L : 0;
        float z[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          z[rr] = sv[rr] * a.scale_log2;
          if ((partial || i >= t_hi) && (t0 + 4 * kq + rr >= t_end)) z[rr] = -INFINITY;
        }
        const float mt = max_over_rows(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
        const float m_new = fmaxf(m, mt);
        const float alpha = exp2_fast(m - m_new);
        float p[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) p[rr] = exp2_fast(z[rr] - (m_new - weight_log2_scale<DT>(0)));
        l = l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
        m = m_new;
#pragma unroll
        for (int u = 0; u < C::kAcc; ++u) acc[u] *= alpha;

        if (partial) {
          // Zero the values of tokens past the end: a NaN there must not reach the sums.
          const bool v0 = t0 + 4 * kq + 0 < L, v1 = t0 + 4 * kq + 1 < L;
          const bool v2 = t0 + 4 * kq + 2 < L, v3 = t0 + 4 * kq + 3 < L;
          if constexpr (DT == kF32) {
            const u4 msk = u4{v0 ? ~0u : 0u, v1 ? ~0u : 0u, v2 ? ~0u : 0u, v3 ? ~0u : 0u};
#pragma unroll
            for (int j = 0; j < C::kLoads; ++j) vb[j] &= msk;
          } else {
            const uint32_t m01 = (v0 ? 0x0000FFFFu : 0u) | (v1 ? 0xFFFF0000u : 0u);
            const uint32_t m23 = (v2 ? 0x0000FFFFu : 0u) | (v3 ? 0xFFFF0000u : 0u);
            const u4 msk = u4{m01, m23, m01, m23};
#pragma unroll
            for (int j = 0; j < C::kLoads; ++j) vb[j] &= msk;
          }
        }

        if constexpr (DT == kF32) {
#pragma unroll
          for (int u = 0; u < C::kLoads; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vb[u][e]), p[e], acc[u], 0, 0, 0);
        } else if constexpr (DT == kBF16) {
          // Value + remainder, each rounded to nearest bf16 (two per packed conversion).
          u2 hb, lb;
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2) {
            hb[i2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{p[2 * i2], p[2 * i2 + 1]}, bf2));
            const float r0 = p[2 * i2] - __uint_as_float(hb[i2] << 16);
            const float r1 = p[2 * i2 + 1] - __uint_as_float(hb[i2] & 0xFFFF0000u);
            lb[i2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{r0, r1}, bf2));
          }
          const s4 ph = __builtin_bit_cast(s4, hb), pl = __builtin_bit_cast(s4, lb);
#pragma unroll
          for (int w = 0; w < C::kLoads; ++w) {
            const s4 a0 = __builtin_bit_cast(s4, u2{vb[w].x, vb[w].y});
            const s4 a1 = __builtin_bit_cast(s4, u2{vb[w].z, vb[w].w});
            acc[2 * w] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a0, ph, acc[2 * w], 0, 0, 0);
            acc[2 * w] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a0, pl, acc[2 * w], 0, 0, 0);
            acc[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a1, ph, acc[2 * w + 1], 0, 0, 0);
            acc[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a1, pl, acc[2 * w + 1], 0, 0, 0);
          }
        } else {
          h4 ph, pl;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const _Float16 hi = (_Float16)p[rr];
            ph[rr] = hi;
            pl[rr] = (_Float16)(p[rr] - (float)hi);
          }
#pragma unroll
          for (int w = 0; w < C::kLoads; ++w) {
            const h4 a0 = __builtin_bit_cast(h4, u2{vb[w].x, vb[w].y});
            const h4 a1 = __builtin_bit_cast(h4, u2{vb[w].z, vb[w].w});
            acc[2 * w] = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, ph, acc[2 * w], 0, 0, 0);
            acc[2 * w] = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, pl, acc[2 * w], 0, 0, 0);
            acc[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, ph, acc[2 * w + 1], 0, 0, 0);
            acc[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, pl, acc[2 * w + 1], 0, 0, 0);
          }
        }
      };

      // Streams tiles [t_lo, t_hi) with cache policy POL. One exit, at the bottom: a tile past
      // t_hi that fills out the last round is loaded from an empty resource (zeros, no memory
      // traffic) and masked out entirely. The next block-table read is issued after the load
      // that uses the previous one, or waiting for that use would also wait for it.
      auto stream = [&](auto pol, int t_lo, int t_hi) {
        int raw_next = bt_entry(t_lo + 1);
        auto issue = [&](int i, u4 (&kb)[C::kLoads], u4 (&vb)[C::kLoads]) {
          load_tile(pol, i, raw_next, t_hi, kb, vb);
          __builtin_amdgcn_sched_barrier(0);
          raw_next = bt_entry(i + 1);
        };
        if constexpr (C::kPrefetch >= 2) {
          // Three register sets in rotation: tiles i+1 and i+2 are in flight while tile i is computed.
          u4 kA[C::kLoads], vA[C::kLoads], kB[C::kLoads], vB[C::kLoads], kC[C::kLoads], vC[C::kLoads];
          int i = t_lo;
          load_tile(pol, i, bt_entry(i), t_hi, kA, vA);
          issue(i + 1, kB, vB);
          do {
            issue(i + 2, kC, vC);
            compute_tile(i, t_hi, kA, vA);
            issue(i + 3, kA, vA);
            compute_tile(i + 1, t_hi, kB, vB);
            issue(i + 4, kB, vB);
            compute_tile(i + 2, t_hi, kC, vC);
            i += 3;
          } while (i < t_hi);
        } else {
          // Two register sets: the loads of tile i+1 are in flight while tile i is computed.
          u4 kA[C::kLoads], vA[C::kLoads], kB[C::kLoads], vB[C::kLoads];
          int i = t_lo;
          load_tile(pol, i, bt_entry(i), t_hi, kA, vA);
          do {
            issue(i + 1, kB, vB);
            compute_tile(i, t_hi, kA, vA);
            issue(i + 2, kA, vA);
            compute_tile(i + 1, t_hi, kB, vB);
            i += 2;
          } while (i < t_hi);
        }
      };
      // Tiles before cached_prefix_tokens with the default policy, the rest streamed: one loop
      // per policy, since a per-tile choice between two load forms defeats the exact waits.
      const int split = min(max((int)(((int64_t)a.cached_prefix_tokens + kTile - 1) / kTile), lt0), lt1);
      if (lt0 < split) stream(std::integral_constant<int, kPolicyDefault>{}, lt0, split);
      if (split < lt1) stream(std::integral_constant<int, kPolicyStream>{}, split, lt1);
    }

    // Sum of the four row groups' partial sums of each head column.
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = (L > 0) ? 1.0f / lt : 0.0f;
    f4 v[C::kAcc];
#pragma unroll
    for (int u = 0; u < C::kAcc; ++u) v[u] = acc[u] * inv;
    if (stash != nullptr) {
      // Rows (row0 + column) of `out` (complete) or of the workspace; every lane writes the same
      // header words and later reads back only what it wrote itself.
      const uint64_t vmask = __ballot(valid);
      const int64_t row0 = complete ? (int64_t)s * a.num_heads + h0 : row_base;
      int* hdr = reinterpret_cast<int*>(stash);
      hdr[0] = (int)row0;
      hdr[1] = (int)(row0 >> 32);
      hdr[2] = (int)vmask;
      hdr[3] = (int)(vmask >> 32);
      hdr[4] = complete ? 1 : 0;
      if (!valid) return;
      // Row-major: column ln's row at float 16 + ln * D, in dim order, so that write_stashed
      // writes whole rows with consecutive lanes on consecutive 16-byte chunks.
      float* rowp = stash + 16 + ln * D;
      if constexpr (DT == kF32) {
#pragma unroll
        for (int u = 0; u < C::kAcc; ++u) *reinterpret_cast<f4*>(rowp + 16 * u + 4 * kq) = v[u];
      } else {
#pragma unroll
        for (int w = 0; w < C::kLoads; ++w) {
          *reinterpret_cast<f4*>(rowp + 32 * w + 8 * kq) = f4{v[2 * w][0], v[2 * w + 1][0], v[2 * w][1], v[2 * w + 1][1]};
          *reinterpret_cast<f4*>(rowp + 32 * w + 8 * kq + 4) =
              f4{v[2 * w][2], v[2 * w + 1][2], v[2 * w][3], v[2 * w + 1][3]};
        }
      }
      if (kq == 0 && !complete) stash[16 + a.ws_cols * D + ln] = m + __log2f(lt);
      return;
    }
    if (!valid) return;

    void* dst = a.out;
    int64_t base;
    bool as_f32 = a.out_f32 != 0;
    if (complete) {
      base = ((int64_t)s * a.num_heads + h0 + ln) * D;
    } else if (part_o != nullptr) {
      dst = part_o;
      base = (int64_t)ln * D;
      as_f32 = true;
      if (kq == 0) part_lse[ln] = m + __log2f(lt);
    } else {
      const int64_t row = row_base + ln;
      dst = a.ws_o;
      base = row * D;
      as_f32 = true;
      if (kq == 0) a.ws_lse[row] = m + __log2f(lt);
    }
    write_row(dst, base, as_f32, v, kq);
  }

  // One lane's share of a head row: normalised O^T tile values v, written from element `base`
  // of dst in fp32 or (as_f32 false) in the input dtype.
  static __device__ __forceinline__ void write_row(void* dst, int64_t base, bool as_f32, const f4 (&v)[C::kAcc],
                                                   int kq) {
    if constexpr (DT == kF32) {
      // O^T tile u holds dims 16u + 4kq + r.
#pragma unroll
      for (int u = 0; u < C::kAcc; ++u)
        *reinterpret_cast<f4*>(reinterpret_cast<float*>(dst) + base + 16 * u + 4 * kq) = v[u];
    } else {
      // O^T tiles 2w (even dims) and 2w+1 (odd dims) hold dims 32w + 8kq + 2r + parity.
#pragma unroll
      for (int w = 0; w < C::kLoads; ++w) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = v[2 * w + (j & 1)][j >> 1];
        store8<DT>(dst, base + 32 * w + 8 * kq, x, as_f32);
      }
    }
  }

  // Writes the rows and segment records that run left in `used` LDS slots: each row in order,
  // consecutive lanes on consecutive 16-byte chunks.
  static __device__ __forceinline__ void write_stashed(const DecodeArgs& a, const float* slots, int used, int lane) {
    constexpr int kChunks = D / 4;  // 16-byte chunks of fp32 per row
    const int cols = a.ws_cols;
    for (int k = 0; k < used; ++k) {
      const float* sl = slots + (int64_t)k * a.stash_slot_floats;
      const int* hdr = reinterpret_cast<const int*>(sl);
      const uint64_t meta = (uint64_t)(uint32_t)hdr[6] | ((uint64_t)(uint32_t)hdr[7] << 32);
      if (meta != 0 && lane == 0) *reinterpret_cast<int4*>(meta) = make_int4(hdr[8], hdr[9], hdr[10], hdr[11]);
      const uint64_t vmask = (uint64_t)(uint32_t)hdr[2] | ((uint64_t)(uint32_t)hdr[3] << 32);
      const int64_t row0 = (int64_t)(uint32_t)hdr[0] | ((int64_t)hdr[1] << 32);
      const bool complete = hdr[4] != 0;
      // Output rows of fp32 inputs are always fp32; workspace rows are fp32.
      const bool as_f32 = !complete || a.out_f32 != 0 || DT == kF32;
      void* dst = complete ? a.out : static_cast<void*>(a.ws_o);
      for (int i = lane; i < cols * kChunks; i += 64) {
        const int c = i / kChunks;
        if (!((vmask >> c) & 1)) continue;
        const int d = (i - c * kChunks) * 4;
        const f4 x = *reinterpret_cast<const f4*>(sl + 16 + c * D + d);
        const int64_t o = (row0 + c) * D + d;
        if (as_f32) {
          *reinterpret_cast<f4*>(reinterpret_cast<float*>(dst) + o) = x;
        } else {
          const float y[4] = {x[0], x[1], x[2], x[3]};
          store4<DT>(dst, o, y, false);
        }
      }
      if (!complete && lane < cols && ((vmask >> lane) & 1)) a.ws_lse[row0 + lane] = sl[16 + cols * D + lane];
    }
  }
};

#ifndef PA_XCD_REMAP
#define PA_XCD_REMAP 1
#endif

// Context length of sequence s, read together with the first lines of its block-table row.
// Entries 0, 16 and 31 (clamped to the row) are read only to bring their lines into the scalar
// cache, so the segment's first block-table reads hit there instead of going to memory after
// the context length has arrived: two dependent memory round trips at a segment's start become
// one. An empty asm statement after the length's clamp consumes them, which keeps the reads and
// places their wait beside the length's own.
__device__ __forceinline__ int seq_len_and_table_lines(const DecodeArgs& a, int s, int max_len) {
  const_i32* row = (const_i32*)(a.block_tables + (int64_t)s * a.max_blocks);
  const int last = a.max_blocks - 1;
  const int b0 = row[0], b1 = row[min(16, last)], b2 = row[min(31, last)];
  const int L = clamp_len(a.context_lens[s], max_len);
  asm volatile("" ::"s"(b0), "s"(b1), "s"(b2));
  return L;
}

// SHARED: the call reads shared prefixes (split modes only); a separate instance keeps that
// bookkeeping out of the plain kernel's walk over its ranges.
template <int DT, int D, bool FUSE, bool SHARED>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(const DecodeArgs a) {
  // Split modes: [num_seqs + 1], the first global tile of each sequence. Workgroup split: the
  // partial rows of the segment being merged.
  extern __shared__ __align__(16) int32_t s_prefix[];
  __shared__ int32_t s_wsum[kWavesPerGroup];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
#if PA_XCD_REMAP
  // Workgroups are dealt round-robin to the 8 XCDs; renumber them so that consecutive
  // ranges (neighbouring sequences, e.g. a prefix-sharing group) run on the same XCD.
  int grp = blockIdx.x;
  if ((gridDim.x & 7) == 0) grp = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int wave = grp * kWavesPerGroup + __builtin_amdgcn_readfirstlane(tid >> 6);
#else
  const int wave = blockIdx.x * kWavesPerGroup + __builtin_amdgcn_readfirstlane(tid >> 6);
#endif
  const int max_len = a.max_blocks << a.bs_log2;
  const int H = a.segs_per_seq;

  if (a.range_tiles == kWorkgroupSplit) {
    // Workgroup split: a workgroup takes whole segments, and its wavefronts stream equal shares
    // of the segment's tiles at once. Each share leaves its normalised partial output and
    // log2-sum-exp2 in LDS, and the workgroup merges them there: no workspace, no second kernel.
    // A one-tile segment is finished by wavefront 0 alone.
    float* part_o = reinterpret_cast<float*>(s_prefix);            // [kWavesPerGroup][gh_max][D]
    float* part_lse = part_o + kWavesPerGroup * a.gh_max * D;      // [kWavesPerGroup][gh_max]
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nseg = a.num_seqs * H;
#if PA_XCD_REMAP
    const int first = grp;
#else
    const int first = blockIdx.x;
#endif
    for (int seg = first; seg < nseg; seg += gridDim.x) {
      const int s = seg / H;
      const int r = seg - s * H;
      const int L = seq_len_and_table_lines(a, s, max_len);
      const int tiles = max(1, (L + kTile - 1) / kTile);
      const int parts = min(kWavesPerGroup, tiles);
      if (parts == 1) {
        if (wv == 0) Piece<DT, D, FUSE>::run(a, s, r, L, 0, tiles, true, 0, lane);
        continue;
      }
      // Every share is non-empty and starts below L, so every partial has a finite lse.
      if (wv < parts)
        Piece<DT, D, FUSE>::run(a, s, r, L, wv * tiles / parts, (wv + 1) * tiles / parts, false, 0, lane,
                                part_o + wv * a.gh_max * D, part_lse + wv * a.gh_max);
      __syncthreads();
      const int g = r / a.n_hg;
      const int hg = r - g * a.n_hg;
      const int h0 = g * a.group + hg * kHeadsPerTile;
      const int gh = min(kHeadsPerTile, a.group - hg * kHeadsPerTile);
      // out = sum_w 2^(lse_w - M) o_w / sum_w 2^(lse_w - M), M = max_w lse_w, shares in order.
      for (int e = tid; e < gh * D; e += kDecodeThreads) {
        const int h = e / D;
        const int d = e - h * D;
        float M = -INFINITY;
        for (int w = 0; w < parts; ++w) M = fmaxf(M, part_lse[w * a.gh_max + h]);
        float num = 0.f, den = 0.f;
        for (int w = 0; w < parts; ++w) {
          const float wt = exp2_fast(part_lse[w * a.gh_max + h] - M);
          den += wt;
          num += wt * part_o[(w * a.gh_max + h) * D + d];
        }
        const float v = num / den;
        const int64_t o = ((int64_t)s * a.num_heads + h0 + h) * D + d;
        if (a.out_f32) {
          reinterpret_cast<float*>(a.out)[o] = v;
        } else if constexpr (DT == kBF16) {
          reinterpret_cast<uint16_t*>(a.out)[o] = (uint16_t)bf16_bits_rne(v);
        } else if constexpr (DT == kF16) {
          reinterpret_cast<_Float16*>(a.out)[o] = (_Float16)v;
        }
      }
      // The next segment's shares overwrite these rows.
      __syncthreads();
    }
    return;
  }

  if (a.range_tiles < 0) {
    // One pass: each wavefront takes whole segments.
    const int nseg = a.num_seqs * H;
    for (int seg = wave; seg < nseg; seg += a.num_waves) {
      const int s = seg / H;
      const int r = seg - s * H;
      const int L = seq_len_and_table_lines(a, s, max_len);
      const int tiles = max(1, (L + kTile - 1) / kTile);
      Piece<DT, D, FUSE>::run(a, s, r, L, 0, tiles, true, 0, lane);
    }
    return;
  }

  // Prefix sums of tiles per sequence (every segment has at least one tile,
  // so an empty sequence still gets a wavefront that writes its zeros).
  // Shared prefixes: a sequence in a group reads only the tiles after the group's prefix, and
  // the group's leader also owns the prefix segments (one per kv head), ahead of its own.
  const int CW = SHARED ? a.casc_width : 0;
  int32_t* s_share = s_prefix + a.num_seqs + 1;  // [num_seqs] sharing words (CW > 0)
  int carry = 0;
  for (int base = 0; base < a.num_seqs; base += kDecodeThreads) {
    const int i = base + tid;
    int v = 0;
    if (i < a.num_seqs) {
      const int L = clamp_len(a.context_lens[i], max_len);
      int tiles = max(1, (L + kTile - 1) / kTile);
      if (CW > 0) {
        const int w = a.ws_share[i];
        s_share[i] = w;
        if (w & kShareIncluded) {
          const int pt = share_tiles(w);
          tiles -= (i % CW == share_leader(w)) ? 0 : pt;
        }
      }
      v = tiles * H;
    }
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wsum[tid >> 6] = x;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerGroup; ++w) {
      const int sw = s_wsum[w];
      before += (w < (tid >> 6)) ? sw : 0;
      total += sw;
    }
    if (i < a.num_seqs) s_prefix[i + 1] = carry + before + x;
    carry += total;
    __syncthreads();
  }
  if (tid == 0) s_prefix[0] = 0;
  __syncthreads();

  const int total = s_prefix[a.num_seqs];
  int R;
  if (a.range_tiles > 0) {
    R = a.range_tiles;
  } else {
    const int n_eff = min(a.num_waves, max(1, (total + kMinTilesPerWave - 1) / kMinTilesPerWave));
    R = (total + n_eff - 1) / n_eff;
  }
  // Ranges are numbered in tile order; range rho covers tiles [rho*R, rho*R + R). In the
  // balanced mode there are at most as many ranges as wavefronts; a fixed range size can
  // need more, and then each wavefront takes every num_waves-th range.
  const int nranges = (total + R - 1) / R;
  // This wavefront's LDS slots for finished rows, written after its last tile.
  float* const slots = reinterpret_cast<float*>(s_prefix) + a.stash_off +
                       __builtin_amdgcn_readfirstlane(tid >> 6) * a.stash_slots * a.stash_slot_floats;
  int used = 0;
  for (int rho = wave; rho < nranges; rho += a.num_waves) {
    int t = rho * R;
    const int t_end = min(total, t + R);

    // Sequence holding tile t: largest s with s_prefix[s] <= t.
    int lo = 0, hi = a.num_seqs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_prefix[mid] <= t) lo = mid; else hi = mid;
    }
    int s = lo;
    // Sequence s's segments, in tile order: pre_tiles-tile prefix segments r = 0..H-1 (a group
    // leader only), then its own segments r = 0..H-1, tiles [skip, skip + own) of the context.
    int L, pre_tiles, skip, own, word;
    auto enter = [&]() {
      L = clamp_len(a.context_lens[s], max_len);
      word = CW > 0 ? s_share[s] : 0;
      skip = (word & kShareIncluded) ? share_tiles(word) : 0;
      pre_tiles = ((word & kShareIncluded) && s % CW == share_leader(word)) ? skip : 0;
      own = max(1, (L + kTile - 1) / kTile - skip);
    };
    enter();
    int local = t - s_prefix[s];
    bool in_pre = local < H * pre_tiles;
    if (!in_pre) local -= H * pre_tiles;
    int r = local / (in_pre ? pre_tiles : own);
    int lt = local - r * (in_pre ? pre_tiles : own);
    bool first = true;
    while (true) {
      const int tiles = in_pre ? pre_tiles : own;
      const int n = min(tiles - lt, t_end - t);
      const int slot = first ? 0 : 1;
      // A piece cut by a range boundary is the range's first (slot 0) or last (slot 1). A whole
      // segment is finished here, unless it belongs to a shared-prefix group (a prefix segment,
      // or a member's own tiles): the merge adds the prefix's partials, so it leaves one partial
      // in rows of its own.
      const bool whole = lt == 0 && n == tiles;
      const bool complete = whole && !in_pre && word == 0;
      int64_t row_base = ((int64_t)rho * 2 + slot) * a.ws_cols;
      if (whole && in_pre) row_base = a.whole_pre_row + ((int64_t)(s / CW) * H + r) * kHeadsPerTile;
      else if (whole) row_base = a.whole_own_row + ((int64_t)s * H + r) * a.gh_max;
      float* stash = used < a.stash_slots ? slots + used * a.stash_slot_floats : nullptr;
      if (lt == 0) {
        // This range holds the segment's first piece: record where all pieces are.
        int4* meta = in_pre ? a.ws_meta_pre + (int64_t)(s / CW) * H + r : a.ws_meta + (int64_t)s * H + r;
        const int4 mv = make_int4(rho, slot, (t + tiles - 1) / R, 0);
        if (stash != nullptr) {
          int* hdr = reinterpret_cast<int*>(stash);
          hdr[6] = (int)(uint32_t)reinterpret_cast<uint64_t>(meta);
          hdr[7] = (int)(reinterpret_cast<uint64_t>(meta) >> 32);
          hdr[8] = mv.x;
          hdr[9] = mv.y;
          hdr[10] = mv.z;
          hdr[11] = mv.w;
        } else if (lane == 0) {
          *meta = mv;
        }
      } else if (stash != nullptr) {
        int* hdr = reinterpret_cast<int*>(stash);
        hdr[6] = 0;
        hdr[7] = 0;
      }
      int win = 0, cols = 0, p_len = L, p_lt0 = skip + lt;
      if (in_pre) {
        // The window's group members: the sequences whose word marks them included.
        win = s - s % CW;
        for (int m = 0; m < CW && win + m < a.num_seqs; ++m)
          cols |= ((s_share[win + m] & kShareIncluded) ? 1 : 0) << m;
        p_len = pre_tiles * kTile;
        p_lt0 = lt;
      }
      Piece<DT, D, FUSE>::run(a, s, r, p_len, p_lt0, p_lt0 + n, complete, row_base, lane, nullptr, nullptr,
                              win, cols, stash);
      used += stash != nullptr ? 1 : 0;
      t += n;
      if (t >= t_end) break;
      first = false;
      lt = 0;
      if (++r == H) {
        r = 0;
        if (in_pre) {
          in_pre = false;
        } else {
          ++s;
          enter();
          in_pre = pre_tiles > 0;
        }
      }
    }
  }
  Piece<DT, D, FUSE>::write_stashed(a, slots, used, lane);
}

// Shared-prefix detection. Sequences are taken in windows of CW = casc_width consecutive ones
// (CW = 16 / group: the query heads of one kv head of CW sequences fill the 16 columns of a
// matrix-core tile); one workgroup of CW wavefronts per window.
// - A sequence takes part if it has a whole block before the block of its last token (the
//   block holding the last token is the one a decode step writes, so it is never shared).
// - The candidates are the sequences whose first physical block is the window's most common
//   one; the first of them leads.
// - Candidate m shares the leading blocks whose physical ids equal the leader's, counted over
//   the whole blocks before either one's last-token block. Ids are compared as the attention
//   kernel uses them (clamped into the pool), so equal ids mean the same K/V bytes.
// - The prefix is the P blocks that maximise P times the number of non-leader candidates
//   sharing at least P blocks: the reads that reading them once saves. The leader and those
//   candidates form the group, if the prefix is at least two tiles long.
// One word per window sequence: kShareIncluded | leader slot << 16 | prefix tiles, 0 if not in
// the group.
__global__ __launch_bounds__(1024) void share_kernel(const DecodeArgs a) {
  __shared__ int s_blocks[kHeadsPerTile];
  const int CW = a.casc_width;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;  // the window slot this wavefront compares
  const int s0 = blockIdx.x * CW;
  const int n = min(CW, a.num_seqs - s0);
  const int max_len = a.max_blocks << a.bs_log2;
  const int64_t nb_max = a.num_blocks - 1;
  auto blk = [&](int v) -> int { return v < 0 ? 0 : ((int64_t)v > nb_max ? (int)nb_max : v); };
  // Lanes 0..n-1 hold the window's sequences (in every wavefront).
  const int me = min(lane, n - 1);
  const int L = clamp_len(a.context_lens[s0 + me], max_len);
  const int cap = (lane < n && L > 0) ? ((L - 1) >> a.bs_log2) : 0;
  const int first = blk(a.block_tables[(int64_t)(s0 + me) * a.max_blocks]);
  int cnt = 0;
  for (int j = 0; j < n; ++j) {
    const int fj = __shfl(first, j), cj = __shfl(cap, j);
    cnt += (cj > 0 && fj == first) ? 1 : 0;
  }
  // Most candidates, then lowest slot.
  int key = cap > 0 ? cnt * 64 + (63 - lane) : -1;
  for (int off = 32; off >= 1; off >>= 1) key = max(key, __shfl_xor(key, off));
  const int leader = 63 - (key & 63);
  const bool group = key >= 2 * 64;
  const int first_l = __shfl(first, leader), cap_l = __shfl(cap, leader);

  int shared_blocks = 0;
  if (group && wv < n) {
    const int first_m = __shfl(first, wv), cap_m = __shfl(cap, wv);
    if (wv == leader) {
      shared_blocks = cap_l;
    } else if (cap_m > 0 && first_m == first_l) {
      const int lim = min(cap_m, cap_l);  // >= 1, and < max_blocks: every index below is in the row
      const int32_t* rm = a.block_tables + (int64_t)(s0 + wv) * a.max_blocks;
      const int32_t* rl = a.block_tables + (int64_t)(s0 + leader) * a.max_blocks;
      shared_blocks = lim;
      for (int j0 = 0; j0 < lim; j0 += 256) {
        int x[4], y[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int j = min(j0 + 64 * k + lane, lim - 1);
          x[k] = blk(rm[j]);
          y[k] = blk(rl[j]);
        }
        int found = -1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int j = j0 + 64 * k + lane;
          const unsigned long long bad = __ballot(j < lim && x[k] != y[k]);
          if (found < 0 && bad != 0) found = j0 + 64 * k + __builtin_ctzll(bad);
        }
        if (found >= 0) {
          shared_blocks = found;
          break;
        }
      }
    }
  }
  if (lane == 0 && wv < kHeadsPerTile) s_blocks[wv] = shared_blocks;
  __syncthreads();
  if (wv != 0) return;

  const int sh = lane < n ? s_blocks[lane] : 0;
  // Saving of a prefix of sh blocks: sh times the non-leader candidates that share that many.
  int c = 0;
  for (int j = 0; j < n; ++j) {
    const int shj = __shfl(sh, j);
    c += (j != leader && shj > 0 && shj >= sh) ? 1 : 0;
  }
  const bool cand = group && lane < n && lane != leader && sh > 0;
  const int saving = cand ? c * sh : 0;  // <= 15 * max_blocks, no overflow
  int best = saving;
  for (int off = 32; off >= 1; off >>= 1) best = max(best, __shfl_xor(best, off));
  // The lowest slot with the best saving gives the prefix length.
  const unsigned long long at = __ballot(cand && saving == best);
  const int tiles_per_block = a.block_size / kTile;
  int p_blocks = (best > 0 && at != 0) ? __shfl(sh, (int)__builtin_ctzll(at)) : 0;
  p_blocks = min(p_blocks, 0xFFFF / tiles_per_block);
  const int p_tiles = p_blocks * tiles_per_block;
  const bool ok = p_tiles >= 2;
  const bool inc = ok && lane < n && (lane == leader || sh >= p_blocks);
  if (lane < n) a.ws_share[s0 + lane] = inc ? (kShareIncluded | (leader << 16) | p_tiles) : 0;
}

// Fused decode step, split modes: cache write of sequence s's new token (position L-1) for kv
// head g, bit copies from k_new / v_new. The attention kernel already used these values from
// registers; they must be in the cache before the next step.
template <int DT, int D>
__device__ __forceinline__ void store_new_token(const DecodeArgs& a, int s, int g, int lane) {
  using C = Cfg<DT, D>;
  const int max_len = a.max_blocks << a.bs_log2;
  const int L = clamp_len(a.context_lens[s], max_len);
  if (L <= 0) return;
  const int t = L - 1;
  int64_t blk = a.block_tables[(int64_t)s * a.max_blocks + (t >> a.bs_log2)];
  blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
  const int bs = a.block_size;
  const int o = t & (bs - 1);
  const int64_t page_bytes = (int64_t)bs * D * C::kE;
  const int64_t page = (blk * a.num_kv_heads + g) * page_bytes;
  const char* kn = reinterpret_cast<const char*>(a.k_new) + ((int64_t)s * a.k_new_stride + (int64_t)g * D) * C::kE;
  const char* vn = reinterpret_cast<const char*>(a.v_new) + ((int64_t)s * a.v_new_stride + (int64_t)g * D) * C::kE;
  char* kc = reinterpret_cast<char*>(const_cast<void*>(a.k_cache)) + page;
  char* vc = reinterpret_cast<char*>(const_cast<void*>(a.v_cache)) + page;
  // K: chunk c of the row goes to ((c * bs) + o) * 16 bytes into the page.
  for (int c = lane; c < C::kChunks; c += 64)
    *reinterpret_cast<u4*>(kc + ((int64_t)c * bs + o) * 16) = *reinterpret_cast<const u4*>(kn + c * 16);
  // V: dim d goes to element ((o / 4) * D + d) * 4 + o % 4 of the page.
  for (int d = lane; d < D; d += 64) {
    const int64_t el = ((int64_t)(o >> 2) * D + d) * 4 + (o & 3);
    if constexpr (DT == kF32)
      reinterpret_cast<uint32_t*>(vc)[el] = reinterpret_cast<const uint32_t*>(vn)[d];
    else
      reinterpret_cast<uint16_t*>(vc)[el] = reinterpret_cast<const uint16_t*>(vn)[d];
  }
}

// Merge of the pieces of every cut segment: out = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M),
// M = max_p lse_p. One wavefront per (segment, head): lane p holds piece p's lse, the pieces'
// output rows are read eight at a time so their loads are in flight together. Summation order
// is fixed (deterministic). SHARED: the call reads shared prefixes, so a sequence in a group also
// merges its window's prefix pieces; a separate instance keeps that bookkeeping out of the
// plain merge.
template <int DT, int D, bool SHARED>
__global__ __launch_bounds__(256) void reduce_kernel(const DecodeArgs a) {
  constexpr int kPer = D / 64;
  constexpr int kBatch = 8;
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int seg = (int)(item / a.gh_max);
  const int n = (int)(item - (int64_t)seg * a.gh_max);
  if (seg >= a.num_seqs * a.segs_per_seq) return;
  const int r = seg % a.segs_per_seq;
  const int g = r / a.n_hg;
  const int hg = r - g * a.n_hg;
  const int gh = min(kHeadsPerTile, a.group - hg * kHeadsPerTile);
  if (n >= gh) return;
  const int s = seg / a.segs_per_seq;
  if (a.k_new != nullptr && n == 0 && hg == 0) store_new_token<DT, D>(a, s, g, lane);
  const int4 meta = a.ws_meta[seg];
  const int wa = meta.x, slot_a = meta.y, wb = meta.z;
  // A sequence in a shared-prefix group also has the pieces of its window's prefix segment,
  // in column (window slot) * group + n.
  int pa = 0, slot_p = 0, np_pre = 0, col_p = 0;
  if constexpr (SHARED) {
    if (a.ws_share[s] & kShareIncluded) {
      const int4 pm = a.ws_meta_pre[(int64_t)(s / a.casc_width) * a.segs_per_seq + r];
      pa = pm.x;
      slot_p = pm.y;
      np_pre = pm.z - pm.x + 1;
      col_p = (s % a.casc_width) * a.group + n;
    }
  }
  if (wb <= wa && np_pre == 0) return;  // finished inside one range
  const int np_own = wb - wa + 1;
  const int np = np_own + np_pre;
  // Workspace row of piece p: range wa + p, slot slot_a for the first piece, 0 after it. With
  // shared prefixes the prefix's pieces follow the own ones, and a segment left whole in one
  // range has rows of its own. Selects only: a lane-dependent branch here would split the
  // batched loads below.
  const int64_t own_whole = a.whole_own_row + (int64_t)seg * a.gh_max + n;
  const int64_t pre_whole =
      np_pre > 0 ? a.whole_pre_row + ((int64_t)(s / a.casc_width) * a.segs_per_seq + r) * kHeadsPerTile + col_p : 0;
  auto row_of = [&](int p) -> int64_t {
    if constexpr (!SHARED) {
      return ((int64_t)(wa + p) * 2 + (p == 0 ? slot_a : 0)) * a.ws_cols + n;
    } else {
      const bool own = p < np_own;
      const int q = own ? p : p - np_own;
      const int first_slot = own ? slot_a : slot_p;
      const int64_t cut =
          ((int64_t)((own ? wa : pa) + q) * 2 + (q == 0 ? first_slot : 0)) * a.ws_cols + (own ? n : col_p);
      const bool whole = own ? np_own == 1 : np_pre == 1;
      return whole ? (own ? own_whole : pre_whole) : cut;
    }
  };
  // Pieces 0..63's lse and the first kBatch pieces' rows are loaded together: the rows do not
  // depend on the weights, so the merge waits for memory once before its first products.
  float vals[kBatch][kPer];
  auto load_batch = [&](int first, int last) {
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const float* o = a.ws_o + row_of(min(first + b, last)) * D + lane * kPer;
#pragma unroll
      for (int j = 0; j < kPer; ++j) vals[b][j] = o[j];
    }
  };
  const float x_raw = a.ws_lse[row_of(min(lane, np - 1))];
  const float x0 = lane < np ? x_raw : -INFINITY;
  load_batch(0, np - 1);
  float M = x0;
  for (int p = 64 + lane; p < np; p += 64) M = fmaxf(M, a.ws_lse[row_of(p)]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

  float acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = 0.f;
  float wsum = 0.f;
  for (int p0 = 0; p0 < np; p0 += 64) {
    const int p = p0 + lane;
    const float x = p0 == 0 ? x0 : (p < np ? a.ws_lse[row_of(p)] : -INFINITY);
    const float wl = (x == -INFINITY) ? 0.f : exp2_fast(x - M);
    wsum += wl;
    const int cnt = min(64, np - p0);
    for (int k0 = 0; k0 < cnt; k0 += kBatch) {
      if (p0 + k0 != 0) load_batch(p0 + k0, p0 + cnt - 1);
      float wk[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) wk[b] = (k0 + b < cnt) ? __shfl(wl, min(k0 + b, cnt - 1)) : 0.f;
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
#pragma unroll
        for (int j = 0; j < kPer; ++j) acc[j] += wk[b] * vals[b][j];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
  const float inv = 1.0f / wsum;
  const int h0 = g * a.group + hg * kHeadsPerTile;
  const int64_t obase = ((int64_t)s * a.num_heads + h0 + n) * D + lane * kPer;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const float v = acc[k] * inv;
    if (a.out_f32) {
      reinterpret_cast<float*>(a.out)[obase + k] = v;
    } else if constexpr (DT == kBF16) {
      reinterpret_cast<uint16_t*>(a.out)[obase + k] = (uint16_t)bf16_bits_rne(v);
    } else if constexpr (DT == kF16) {
      reinterpret_cast<_Float16*>(a.out)[obase + k] = (_Float16)v;
    }
  }
}

// Fused decode step without the fused attention kernel: the step's token of every (sequence, kv
// head) written to its cache slot (one wavefront each) before the plain kernels run.
template <int DT, int D>
__global__ __launch_bounds__(256) void append_kernel(const DecodeArgs a) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (int64_t)a.num_seqs * a.num_kv_heads) return;
  store_new_token<DT, D>(a, (int)(w / a.num_kv_heads), (int)(w % a.num_kv_heads), threadIdx.x & 63);
}

// Whether the attention kernel takes the step's token itself (fused decode step). At fp32 and
// head_dim 256 the fused instance would hold the token's K/V rows (80 registers) beside the
// tiles' and spill to scratch; there the token is written first (append_kernel).
template <int DT, int D>
constexpr bool kFusedStep = !(DT == kF32 && D == 256);

template <int DT, int D>
hipError_t launch_decode_t(const DecodeArgs& a, int grid, size_t lds, hipStream_t st) {
  const dim3 g(grid), b(kDecodeThreads);
  if constexpr (kFusedStep<DT, D>) {
    if (a.k_new != nullptr) {
      if (a.casc_width > 0)
        hipLaunchKernelGGL((decode_kernel<DT, D, true, true>), g, b, lds, st, a);
      else
        hipLaunchKernelGGL((decode_kernel<DT, D, true, false>), g, b, lds, st, a);
      return hipGetLastError();
    }
  } else {
    if (a.k_new != nullptr) return hipErrorInvalidValue;  // the host writes the token first
  }
  if (a.casc_width > 0)
    hipLaunchKernelGGL((decode_kernel<DT, D, false, true>), g, b, lds, st, a);
  else
    hipLaunchKernelGGL((decode_kernel<DT, D, false, false>), g, b, lds, st, a);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_append_t(const DecodeArgs& a, hipStream_t st) {
  const int64_t waves = (int64_t)a.num_seqs * a.num_kv_heads;
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL((append_kernel<DT, D>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_reduce_t(const DecodeArgs& a, hipStream_t st) {
  const int64_t items = (int64_t)a.num_seqs * a.segs_per_seq * a.gh_max;
  const dim3 grid((unsigned)((items + 3) / 4));
  if (a.casc_width > 0)
    hipLaunchKernelGGL((reduce_kernel<DT, D, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((reduce_kernel<DT, D, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_share_t(const DecodeArgs& a, hipStream_t st) {
  const int windows = (a.num_seqs + a.casc_width - 1) / a.casc_width;
  hipLaunchKernelGGL(share_kernel, dim3(windows), dim3(64 * a.casc_width), 0, st, a);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t occupancy_t(size_t lds, int* groups) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(groups, decode_kernel<DT, D, false, false>, kDecodeThreads, lds);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int grid, size_t lds, hipStream_t st) {
  switch (dtype) {
    case kF32:
      if (head_dim == 64) return launch_decode_t<kF32, 64>(a, grid, lds, st);
      if (head_dim == 128) return launch_decode_t<kF32, 128>(a, grid, lds, st);
      if (head_dim == 256) return launch_decode_t<kF32, 256>(a, grid, lds, st);
      break;
    case kF16:
      if (head_dim == 64) return launch_decode_t<kF16, 64>(a, grid, lds, st);
      if (head_dim == 128) return launch_decode_t<kF16, 128>(a, grid, lds, st);
      if (head_dim == 256) return launch_decode_t<kF16, 256>(a, grid, lds, st);
      break;
    case kBF16:
      if (head_dim == 64) return launch_decode_t<kBF16, 64>(a, grid, lds, st);
      if (head_dim == 128) return launch_decode_t<kBF16, 128>(a, grid, lds, st);
      if (head_dim == 256) return launch_decode_t<kBF16, 256>(a, grid, lds, st);
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_share(const DecodeArgs& a, hipStream_t st) { return launch_share_t(a, st); }

bool decode_fuses_step(int dtype, int head_dim) {
  switch (dtype) {
    case kF32:
      return head_dim == 64 ? kFusedStep<kF32, 64> : head_dim == 128 ? kFusedStep<kF32, 128> : kFusedStep<kF32, 256>;
    case kF16:
      return head_dim == 64 ? kFusedStep<kF16, 64> : head_dim == 128 ? kFusedStep<kF16, 128> : kFusedStep<kF16, 256>;
    default:
      return head_dim == 64 ? kFusedStep<kBF16, 64> : head_dim == 128 ? kFusedStep<kBF16, 128>
                                                                       : kFusedStep<kBF16, 256>;
  }
}

hipError_t launch_append(const DecodeArgs& a, int dtype, int head_dim, hipStream_t st) {
  switch (dtype) {
    case kF32:
      if (head_dim == 64) return launch_append_t<kF32, 64>(a, st);
      if (head_dim == 128) return launch_append_t<kF32, 128>(a, st);
      if (head_dim == 256) return launch_append_t<kF32, 256>(a, st);
      break;
    case kF16:
      if (head_dim == 64) return launch_append_t<kF16, 64>(a, st);
      if (head_dim == 128) return launch_append_t<kF16, 128>(a, st);
      if (head_dim == 256) return launch_append_t<kF16, 256>(a, st);
      break;
    case kBF16:
      if (head_dim == 64) return launch_append_t<kBF16, 64>(a, st);
      if (head_dim == 128) return launch_append_t<kBF16, 128>(a, st);
      if (head_dim == 256) return launch_append_t<kBF16, 256>(a, st);
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_reduce(const DecodeArgs& a, int dtype, int head_dim, hipStream_t st) {
  switch (dtype) {
    case kF32:
      if (head_dim == 64) return launch_reduce_t<kF32, 64>(a, st);
      if (head_dim == 128) return launch_reduce_t<kF32, 128>(a, st);
      if (head_dim == 256) return launch_reduce_t<kF32, 256>(a, st);
      break;
    case kF16:
      if (head_dim == 64) return launch_reduce_t<kF16, 64>(a, st);
      if (head_dim == 128) return launch_reduce_t<kF16, 128>(a, st);
      if (head_dim == 256) return launch_reduce_t<kF16, 256>(a, st);
      break;
    case kBF16:
      if (head_dim == 64) return launch_reduce_t<kBF16, 64>(a, st);
      if (head_dim == 128) return launch_reduce_t<kBF16, 128>(a, st);
      if (head_dim == 256) return launch_reduce_t<kBF16, 256>(a, st);
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t decode_groups_per_cu(int dtype, int head_dim, size_t lds, int* groups) {
  switch (dtype) {
    case kF32:
      if (head_dim == 64) return occupancy_t<kF32, 64>(lds, groups);
      if (head_dim == 128) return occupancy_t<kF32, 128>(lds, groups);
      if (head_dim == 256) return occupancy_t<kF32, 256>(lds, groups);
      break;
    case kF16:
      if (head_dim == 64) return occupancy_t<kF16, 64>(lds, groups);
      if (head_dim == 128) return occupancy_t<kF16, 128>(lds, groups);
      if (head_dim == 256) return occupancy_t<kF16, 256>(lds, groups);
      break;
    case kBF16:
      if (head_dim == 64) return occupancy_t<kBF16, 64>(lds, groups);
      if (head_dim == 128) return occupancy_t<kBF16, 128>(lds, groups);
      if (head_dim == 256) return occupancy_t<kBF16, 256>(lds, groups);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
