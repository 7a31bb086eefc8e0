// Paged prefill for gfx950: causal attention of each sequence's new tokens
// over its paged KV cache (flash-attention prefill with online softmax,
// miniVLLM docs, "What is miniVLLM?" and "Explore by topic"; hysenlabs MinivLLM
// review, prefilling-baseline section).
//
// Sequence s has n new query tokens (rows query_start[s] .. query_start[s+1]-1
// of q) at positions L-n .. L-1 of its L cached tokens; query i attends to
// tokens 0 .. L-n+i. n = L is an ordinary prefill, n < L a prefill after a
// prefix-cache hit or a chunk of a chunked prefill, n = 1 a decode step.
//
// Work item: (sequence, kv head, head group, block of queries). One wavefront
// streams the sequence's K/V up to the block's last query and keeps, per
// column, an online-softmax state. The 16 columns of a matrix-core tile are
// (query, head) pairs: 16/G queries x G heads of one kv head (or 16 heads of
// one query when G > 16). Several column tiles share each K/V load (more at
// smaller head_dim and 16-bit inputs, where registers allow).
//
// The key stream advances 32 tokens (two 16-token tiles A and B) per step:
//   S_A, S_B = K_{A,B} . Q^T          (rows = tokens, cols = (query, head))
//   one online-softmax update over the step's 32 keys per column
//   O^T += V^T . P^T                  (contraction over the step's 32 keys)
// For 16-bit inputs the second product is one 32-deep matrix-core
// instruction per 16 output rows. Its contraction index runs over the 32 keys
// in the order (A: 4kq..4kq+3, B: 4kq..4kq+3) for lane group kq, which is the
// order in which the first product leaves P in registers; V^T's operand takes
// the same order from the two tiles' V loads. For bf16, P enters as a sum of
// two bf16 parts, value + remainder, each rounded to nearest (relative error
// <= 2^-16). For fp16, P enters once, rounded to nearest (<= 2^-11), and the
// softmax denominator sums those same rounded weights; one fp16 rounding keeps
// the output within the tolerance with a wide margin, where one bf16 rounding
// (2^-9) would not.
//
// K of the next step is requested as soon as this step's scores are issued,
// V of the next step as soon as this step's second product is issued. Every
// query block of a sequence re-reads the same keys, so the loads use the
// default (caching) policy.
//
// Two kernels share this scheme. prefill_kernel gives each wavefront its own
// item and its own K/V loads. prefill_shared_kernel (16-bit inputs at
// head_dim 128) gives a workgroup four consecutive query blocks; each 32-key
// step is loaded once per workgroup, a quarter by each wavefront, and read by
// all four from LDS. Both take their items from per-XCD work queues
// (WorkQueue below), so no workgroup ends with much more work than the others.

#include "device_common.h"

#include <float.h>

namespace pa {
namespace {

using namespace dev;

#ifndef PA_PREFILL_NC64
#define PA_PREFILL_NC64 4
#endif
#ifndef PA_PREFILL_NC128
#define PA_PREFILL_NC128 2
#endif

// Column tiles per wavefront: every K/V load serves 16 * col_tiles columns.
constexpr int prefill_col_tiles(int dtype, int head_dim) {
  return dtype == kF32 ? (head_dim <= 64 ? 2 : 1)
                       : (head_dim <= 64 ? PA_PREFILL_NC64 : (head_dim <= 128 ? PA_PREFILL_NC128 : 1));
}

template <int DT, int D>
struct PrefillCfg {
  using C = Cfg<DT, D>;
  static constexpr int kNC = prefill_col_tiles(DT, D);
};


// Sequence s's context length L and its new query rows q0 .. q0+n-1, with every value read
// from device memory clamped into what the call describes: L into [0, max_len], the rows into
// [0, num_tokens) and n into [0, L]. No query_start or context_lens content can move a q read or
// an out write outside the buffers.
__device__ __forceinline__ void seq_rows(const PrefillArgs& a, int s, int& L, int& q0, int& n) {
  const int max_len = a.max_blocks << a.bs_log2;
  L = a.context_lens[s];
  L = L < 0 ? 0 : (L > max_len ? max_len : L);
  int b = a.query_start[s], e = a.query_start[s + 1];
  b = b < 0 ? 0 : (b > a.num_tokens ? a.num_tokens : b);
  e = e < b ? b : (e > a.num_tokens ? a.num_tokens : e);
  q0 = b;
  n = e - b < L ? e - b : L;
}

template <int DT, int D>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, int s, int g, int hg, int qb, int lane) {
  using C = Cfg<DT, D>;
  constexpr int NC = PrefillCfg<DT, D>::kNC;
  const int kq = lane >> 4;
  const int ln = lane & 15;
  const int bs = a.block_size;
  int L, q0, n;
  seq_rows(a, s, L, q0, n);
  const int gh = a.gh_max;            // columns per query (heads of one group)
  const int qpt = kHeadsPerTile / gh; // queries per column tile
  const int qb_queries = NC * qpt;
  const int qfirst = qb * qb_queries;
  if (qfirst >= n) return;
  const int qlast = min(n, qfirst + qb_queries) - 1;
  const int p_first = L - n + qfirst;  // position of the block's first query
  const int p_last = L - n + qlast;

  // Column (ct, ln): query qi, head h; padding columns get q = 0 and the last position.
  int qi[NC], hh[NC], pos[NC];
  bool valid[NC];
#pragma unroll
  for (int ct = 0; ct < NC; ++ct) {
    const int ql = ln / gh;
    const int hl = hg * kHeadsPerTile + (ln % gh);
    qi[ct] = qfirst + ct * qpt + ql;
    hh[ct] = g * a.group + hl;
    valid[ct] = ql < qpt && hl < a.group && qi[ct] < n;
    pos[ct] = valid[ct] ? L - n + qi[ct] : p_last;
  }
  // Logits in the log2 domain are c * (q . k) with c = |scale| * log2(e) > 0: a negative scale
  // moves its sign into q (a sign flip, exact), and a zero scale becomes the smallest normal
  // number, which gives the same equal weights. With c > 0 the scaling folds into exp2's
  // argument and masked keys (-inf) stay -inf.
  const uint32_t qflip = a.scale_log2 < 0.f ? (DT == kF32 ? 0x80000000u : 0x80008000u) : 0u;
  const float c = fmaxf(fabsf(a.scale_log2), FLT_MIN);
  u4 qv[NC][C::kLoads];
#pragma unroll
  for (int ct = 0; ct < NC; ++ct) {
    const char* qrow = reinterpret_cast<const char*>(a.q) +
                       ((int64_t)(q0 + qi[ct]) * a.q_token_stride + (int64_t)hh[ct] * D) * C::kE;
#pragma unroll
    for (int j = 0; j < C::kLoads; ++j) {
      qv[ct][j] = valid[ct] ? *reinterpret_cast<const u4*>(qrow + (4 * j + kq) * 16) : u4{0u, 0u, 0u, 0u};
      qv[ct][j] ^= u4{qflip, qflip, qflip, qflip};
    }
  }

  f4 acc[NC][C::kAcc];
  f4 accl[NC];  // fp16: running sums of the rounded weights (matrix cores; every row the same)
  float m[NC], l[NC];
  float thr[NC];  // (m + 8) / c: a raw score above it moves the running maximum
#pragma unroll
  for (int ct = 0; ct < NC; ++ct) {
    m[ct] = -INFINITY;
    thr[ct] = -INFINITY;
    l[ct] = 0.f;
#pragma unroll
    for (int u = 0; u < C::kAcc; ++u) acc[ct][u] = f4{0.f, 0.f, 0.f, 0.f};
    accl[ct] = f4{0.f, 0.f, 0.f, 0.f};
  }
  // Matrix-core weight sums (fp16): an all-ones operand, kept in registers.
  u4 ones_u = u4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
  asm volatile("" : "+v"(ones_u));
  const h8 ones8 = __builtin_bit_cast(h8, ones_u);
  (void)ones8;

  const int64_t page_bytes = (int64_t)bs * D * C::kE;
  const int page_bytes32 = (int)page_bytes;
  const int64_t blk_stride = (int64_t)a.num_kv_heads * page_bytes;
  const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (int64_t)g * page_bytes;
  const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (int64_t)g * page_bytes;
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;
  // Block ids are int32: clamped in 32 bits, into [0, num_blocks - 1].
  const int nb_max = (int)(a.num_blocks - 1 < INT32_MAX ? a.num_blocks - 1 : INT32_MAX);
  // Lane offsets inside a page. K: chunk (4j + kq) of token (off0 + ln). V, 16-bit: 8 bytes =
  // tokens off0 + 4kq .. +3 of dim 32w + ln (and of dim 32w + 16 + ln at +128 bytes). V, fp32:
  // 16 bytes = tokens off0 + 4kq .. +3 of dim 16u + ln.
  const uint32_t k_lane = (uint32_t)((kq * bs + ln) * 16);
  const uint32_t v_lane = (DT == kF32) ? (uint32_t)((kq * D + ln) * 16) : (uint32_t)((kq * D + ln) * 8);

  // Keys 0 .. p_last in 16-token tiles, two per step. Tile indices are clamped to the last
  // tile, so every step issues the same loads: the second tile of an odd last step re-reads
  // the first (it is masked), and the loop's final prefetch re-reads the last step. With no
  // conditional load in the loop, the compiler's wait counts stay exact and the next step's
  // loads overlap this step's arithmetic.
  const int tiles = p_last / kTile + 1;
  const int steps = (tiles + 1) >> 1;
  auto tile_of = [&](int st, int half) { return min(2 * st + half, tiles - 1); };
  // Block-table entries of a step's two tiles: two scalar loads, issued two steps ahead.
  const_i32* cbt = (const_i32*)bt;
  auto bt_load = [&](int st) -> int2 {
    const int sc = min(st, steps - 1);
    return make_int2(cbt[(tile_of(sc, 0) * kTile) >> a.bs_log2], cbt[(tile_of(sc, 1) * kTile) >> a.bs_log2]);
  };
  auto block = [&](int raw) -> int64_t {
    const int b = __builtin_amdgcn_readfirstlane(raw);
    return (int64_t)min(max(b, 0), nb_max);
  };
  u4 kA[C::kLoads], kB[C::kLoads];
  // 16-bit: vr0[w] / vr1[w] are the second product's V^T operands for dims 32w + ln /
  // 32w + 16 + ln, keys in P's slot order (tile A's four, then tile B's four).
  // fp32: vr0 / vr1 are tile A's / tile B's 16-byte loads.
  u4 vr0[C::kLoads], vr1[C::kLoads];
  auto issue_k = [&](int st, int64_t ba, int64_t bb) {
    const int sc = min(st, steps - 1);
    const __amdgpu_buffer_rsrc_t ra = page_rsrc(kbase + ba * blk_stride, page_bytes32);
    const __amdgpu_buffer_rsrc_t rb = page_rsrc(kbase + bb * blk_stride, page_bytes32);
    const int oa = (int)k_lane + ((tile_of(sc, 0) * kTile) & (bs - 1)) * 16;
    const int ob = (int)k_lane + ((tile_of(sc, 1) * kTile) & (bs - 1)) * 16;
#pragma unroll
    for (int j = 0; j < C::kLoads; ++j) kA[j] = buf_load16<kPolicyDefault>(ra, oa + j * 64 * bs);
#pragma unroll
    for (int j = 0; j < C::kLoads; ++j) kB[j] = buf_load16<kPolicyDefault>(rb, ob + j * 64 * bs);
  };
  auto issue_v = [&](int st, int64_t ba, int64_t bb) {
    const int sc = min(st, steps - 1);
    const __amdgpu_buffer_rsrc_t ra = page_rsrc(vbase + ba * blk_stride, page_bytes32);
    const __amdgpu_buffer_rsrc_t rb = page_rsrc(vbase + bb * blk_stride, page_bytes32);
    const int oa = (int)v_lane + ((tile_of(sc, 0) * kTile) & (bs - 1)) * D * C::kE;
    const int ob = (int)v_lane + ((tile_of(sc, 1) * kTile) & (bs - 1)) * D * C::kE;
    if constexpr (DT == kF32) {
#pragma unroll
      for (int j = 0; j < C::kLoads; ++j) vr0[j] = buf_load16<kPolicyDefault>(ra, oa + j * 256);
#pragma unroll
      for (int j = 0; j < C::kLoads; ++j) vr1[j] = buf_load16<kPolicyDefault>(rb, ob + j * 256);
    } else {
#pragma unroll
      for (int w = 0; w < C::kLoads; ++w) {
        const u2 a0 = buf_load8<kPolicyDefault>(ra, oa + w * 256);
        const u2 a1 = buf_load8<kPolicyDefault>(ra, oa + w * 256 + 128);
        const u2 b0 = buf_load8<kPolicyDefault>(rb, ob + w * 256);
        const u2 b1 = buf_load8<kPolicyDefault>(rb, ob + w * 256 + 128);
        vr0[w] = u4{a0[0], a0[1], b0[0], b0[1]};
        vr1[w] = u4{a1[0], a1[1], b1[0], b1[1]};
      }
    }
  };
  // Zero the values of keys at or beyond L (their slots may hold anything, and a zero weight
  // times a NaN is still NaN) and of a second tile that does not exist.
  auto mask_v = [&](int t0, bool has_b) {
    // Only a sequence's last step reaches past L: a wave-uniform branch, kept as one (else the
    // compiler turns it into selects and masks that every step would pay for).
    const int full = __builtin_amdgcn_readfirstlane((t0 + 2 * kTile <= L && has_b) ? 1 : 0);
    if (__builtin_expect(full != 0, 1)) return;
    uint32_t mk[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) mk[h][e] = (h == 0 || has_b) && t0 + h * kTile + 4 * kq + e < L ? ~0u : 0u;
    if constexpr (DT == kF32) {
#pragma unroll
      for (int j = 0; j < C::kLoads; ++j) {
        vr0[j] &= u4{mk[0][0], mk[0][1], mk[0][2], mk[0][3]};
        vr1[j] &= u4{mk[1][0], mk[1][1], mk[1][2], mk[1][3]};
      }
    } else {
      const u4 msk = u4{(mk[0][0] & 0xFFFFu) | (mk[0][1] & 0xFFFF0000u), (mk[0][2] & 0xFFFFu) | (mk[0][3] & 0xFFFF0000u),
                        (mk[1][0] & 0xFFFFu) | (mk[1][1] & 0xFFFF0000u), (mk[1][2] & 0xFFFFu) | (mk[1][3] & 0xFFFF0000u)};
#pragma unroll
      for (int w = 0; w < C::kLoads; ++w) {
        vr0[w] &= msk;
        vr1[w] &= msk;
      }
    }
  };
  auto scores = [&](const u4 (&kb)[C::kLoads], const u4 (&q)[C::kLoads]) -> f4 {
    f4 sv = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < C::kLoads; ++j) {
      if constexpr (DT == kF32) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sv = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kb[j][e]), __uint_as_float(q[j][e]), sv, 0, 0, 0);
      } else if constexpr (DT == kBF16) {
        sv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, kb[j]), __builtin_bit_cast(b8, q[j]), sv,
                                                     0, 0, 0);
      } else {
        sv = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, kb[j]), __builtin_bit_cast(h8, q[j]), sv,
                                                    0, 0, 0);
      }
    }
    return sv;
  };

  // Step -1 only issues the loads of step 0, from the same code as every later prefetch, so
  // the compiler sees one load order and keeps its waits exact.
  int2 bt_next = bt_load(0);
  for (int st = -1; st < steps; ++st) {
    const int t0 = st * 2 * kTile;
    const bool has_b = 2 * st + 1 < tiles;
    f4 sA[NC], sB[NC];
    if (st >= 0) {
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        sA[ct] = scores(kA, qv[ct]);
        sB[ct] = scores(kB, qv[ct]);
      }
    }
    const int64_t nA = block(bt_next.x), nB = block(bt_next.y);
    bt_next = bt_load(st + 2);
    issue_k(st + 1, nA, nB);
    // K before V in every copy of this code the compiler makes (it peels step -1).
    __builtin_amdgcn_sched_barrier(0);
    if (st < 0) {
      issue_v(0, nA, nB);
      continue;
    }
    mask_v(t0, has_b);
    // every key of the step visible to every column: no masking
    const bool open = t0 + 2 * kTile - 1 <= p_first;

    // Both wave-uniform branches of the step (the causal mask, the rescale) are taken once for
    // all column tiles. The exponentials, weight splits and second products of all tiles then
    // form one branch-free block, in which the compiler can interleave one tile's products with
    // the next tile's softmax.
    float x[NC][8];
#pragma unroll
    for (int ct = 0; ct < NC; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[ct][r] = sA[ct][r];
        x[ct][4 + r] = sB[ct][r];
      }
    if (!open) {
#pragma unroll
      for (int ct = 0; ct < NC; ++ct)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = t0 + (j < 4 ? 0 : kTile) + 4 * kq + (j & 3);
          if (t > pos[ct]) x[ct][j] = -INFINITY;
        }
    }
    // The running maximum m of each column is kept unless a score exceeds it by more than 8
    // (log2 units): weights stay below 2^8, and the accumulators are rescaled only on such
    // jumps. Each lane tests its own raw scores against thr = (m + 8) / c (c > 0), kept with m,
    // so the test costs no arithmetic per score; only when some lane finds a jump is the
    // maximum over the column's rows taken. That happens on an item's first step (m = -inf; key
    // 0 is visible to every column, so m is finite afterwards) and on real jumps. Columns
    // without a jump keep alpha = 1. Where x > thr and x * c > m + 8 disagree (within a rounding
    // of the threshold) either no rescale happens and a weight exceeds 2^8 by a rounding, or
    // the rescale finds m + 8 not exceeded and keeps m: both harmless.
    float alpha[NC];
    bool jump = false;
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
      alpha[ct] = 1.0f;
      // IEEE-2019 maximum: gfx950 has a three-input form, and it needs no NaN quieting first.
      // Bitwise or: a short-circuit || would become a masked branch per column tile. The bf16
      // head_dim-64 instance keeps ||: straight-line, its registers overflow into AGPRs and it
      // drops to one wavefront per SIMD.
      if constexpr (DT == kBF16 && D == 64) jump = jump || fmax8(x[ct]) > thr[ct];
      else jump = jump | (fmax8(x[ct]) > thr[ct]);
    }
    if (__builtin_amdgcn_ballot_w64(jump) != 0) {
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        const float mt = max_over_rows(fmax8(x[ct]));
        const float m_cand = __builtin_elementwise_maximum(m[ct], mt * c);
        const float m_use = m_cand > m[ct] + 8.0f ? m_cand : m[ct];
        alpha[ct] = exp2_fast(m[ct] - m_use);
        m[ct] = m_use;
        thr[ct] = (m_use + 8.0f) / c;
#pragma unroll
        for (int u = 0; u < C::kAcc; ++u) acc[ct][u] *= alpha[ct];
        accl[ct] *= alpha[ct];
      }
    }

#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = exp2_fast(fmaf(x[ct][j], c, weight_log2_scale<DT>(8) - m[ct]));
      // fp16: the running sum is taken over the rounded weights, on the matrix cores (below)
      if constexpr (DT != kF16)
        l[ct] = fmaf(l[ct], alpha[ct], ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));

      if constexpr (DT == kF32) {
#pragma unroll
        for (int u = 0; u < C::kLoads; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[ct][u] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vr0[u][e]), p[e], acc[ct][u], 0, 0, 0);
            acc[ct][u] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vr1[u][e]), p[4 + e], acc[ct][u], 0, 0, 0);
          }
      } else {
        // P^T operand: slot j of lane group kq = key (j < 4 ? A : B) 4kq + (j & 3).
        u4 ph, pl;  // pl: bf16 remainder parts
        if constexpr (DT == kBF16) {
          // gfx950 rounds two floats to bf16 (nearest even) in one instruction.
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) {
            const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{p[2 * i2], p[2 * i2 + 1]}, bf2));
            const float r0 = p[2 * i2] - __uint_as_float(hb << 16);
            const float r1 = p[2 * i2 + 1] - __uint_as_float(hb & 0xFFFF0000u);
            ph[i2] = hb;
            pl[i2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{r0, r1}, bf2));
          }
        } else {
          // fp16: one part, rounded to nearest (relative error <= 2^-11). The running sum is of
          // exactly these rounded weights, taken on the matrix cores (an all-ones row operand:
          // every output row is the column's sum over the 32 keys, in fp32), so the
          // normalisation matches the product: equal weights, or one dominant weight, give their
          // values' mean exactly.
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2)
            ph[i2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{p[2 * i2], p[2 * i2 + 1]}, hf2));
          accl[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones8, __builtin_bit_cast(h8, ph), accl[ct], 0, 0, 0);
        }
#pragma unroll
        for (int w = 0; w < C::kLoads; ++w) {
          if constexpr (DT == kBF16) {
            const b8 bh = __builtin_bit_cast(b8, ph), bl = __builtin_bit_cast(b8, pl);
            const b8 a0 = __builtin_bit_cast(b8, vr0[w]), a1 = __builtin_bit_cast(b8, vr1[w]);
            acc[ct][2 * w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bh, acc[ct][2 * w], 0, 0, 0);
            acc[ct][2 * w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bl, acc[ct][2 * w], 0, 0, 0);
            acc[ct][2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bh, acc[ct][2 * w + 1], 0, 0, 0);
            acc[ct][2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bl, acc[ct][2 * w + 1], 0, 0, 0);
          } else {
            const h8 hh8 = __builtin_bit_cast(h8, ph);
            const h8 a0 = __builtin_bit_cast(h8, vr0[w]), a1 = __builtin_bit_cast(h8, vr1[w]);
            acc[ct][2 * w] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, hh8, acc[ct][2 * w], 0, 0, 0);
            acc[ct][2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, hh8, acc[ct][2 * w + 1], 0, 0, 0);
          }
        }
      }
    }
    issue_v(st + 1, nA, nB);
  }

  // Output rows: fp32 inputs, acc[u] row i = dim 16u + i; 16-bit inputs, acc[2w] row i =
  // dim 32w + i and acc[2w + 1] row i = dim 32w + 16 + i. Lane (kq, ln) holds rows 4kq .. 4kq+3.
#pragma unroll
  for (int ct = 0; ct < NC; ++ct) {
    float lt;
    if constexpr (DT == kF16) {
      lt = accl[ct][0];  // already summed over all keys (and lane groups) by the matrix cores
    } else {
      lt = l[ct] + __shfl_xor(l[ct], 16);
      lt += __shfl_xor(lt, 32);
    }
    const float inv = 1.0f / lt;
    if (!valid[ct]) continue;
    const int64_t base = ((int64_t)(q0 + qi[ct]) * a.num_heads + hh[ct]) * D;
    if constexpr (DT == kF32) {
#pragma unroll
      for (int u = 0; u < C::kAcc; ++u)
        *reinterpret_cast<f4*>(reinterpret_cast<float*>(a.out) + base + 16 * u + 4 * kq) = acc[ct][u] * inv;
    } else {
#pragma unroll
      for (int w = 0; w < C::kLoads; ++w) {
        const float v0[4] = {acc[ct][2 * w][0] * inv, acc[ct][2 * w][1] * inv, acc[ct][2 * w][2] * inv,
                             acc[ct][2 * w][3] * inv};
        const float v1[4] = {acc[ct][2 * w + 1][0] * inv, acc[ct][2 * w + 1][1] * inv, acc[ct][2 * w + 1][2] * inv,
                             acc[ct][2 * w + 1][3] * inv};
        store4<DT>(a.out, base + 32 * w + 4 * kq, v0, a.out_f32 != 0);
        store4<DT>(a.out, base + 32 * w + 16 + 4 * kq, v1, a.out_f32 != 0);
      }
    }
  }
}

// s_prefix[i] = first work item of sequence i, where a sequence has ceil(n / queries_per_item)
// items per (kv head, head group); n = its new tokens. Returns the total. All threads call it.
__device__ int build_item_prefix(const PrefillArgs& a, int queries_per_item, int32_t* s_prefix, int32_t* s_wsum) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int H = a.num_kv_heads * a.n_hg;
  int carry = 0;
  for (int base = 0; base < a.num_seqs; base += kDecodeThreads) {
    const int i = base + tid;
    int v = 0;
    if (i < a.num_seqs) {
      int L, q0, n;
      seq_rows(a, i, L, q0, n);
      v = ((n + queries_per_item - 1) / queries_per_item) * H;
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
  return s_prefix[a.num_seqs];
}

// Work queues. Items cost from one 32-key step to thousands (a query block's keys run up to its
// last query), so a fixed assignment of items to persistent workgroups leaves some with far more
// work than others: round-robin over the items in their order gives the busiest 1.25-1.5 times
// the mean on long and mixed prompts. Instead each workgroup takes its next item (per-wavefront
// kernel: the next chunk of four, one per wavefront) from a counter when it is free; its first
// one is fixed, so no launch starts by waiting on an atomic. There is one counter per XCD
// (workgroups are dealt to the 8 XCDs round-robin), and the items are dealt to them in chunks of
// kQueueChunk consecutive ones, neighbouring query blocks of one (sequence, kv head) that read
// the same K/V pages, so those stay in one XCD's L2.
// The counters live in a static array, kQueueSlots sets of them; the host gives every call the
// next set. The last workgroup of a launch to finish sets its counters back to zero,
// so every launch (and every replay of a captured one) starts from zero. Nothing waits on another
// workgroup: a launch whose workgroups run one after another is only slower.
constexpr int kQueueChunk = 4;
constexpr int kQueueWords = 16;  // 8 XCD counters, the finished count, padding
__device__ uint32_t g_prefill_queues[kQueueSlots * kQueueWords];

struct WorkQueue {
  uint32_t* ctr;
  int nq, q;
  uint32_t rank, per_queue;  // this workgroup's index among its queue's workgroups, and their count
  __device__ WorkQueue(const PrefillArgs& a) {
    ctr = g_prefill_queues + (uint32_t)a.queue_slot * kQueueWords;
    nq = (gridDim.x & 7) == 0 ? 8 : 1;
    q = (int)(blockIdx.x & (uint32_t)(nq - 1));
    rank = blockIdx.x / (uint32_t)nq;
    per_queue = gridDim.x / (uint32_t)nq;
  }
  // A workgroup's first index is its rank; later ones come from the counter, past the first
  // round. Requests the next index (one lane's atomic; its value is read later).
  __device__ uint32_t request(bool leader) const { return leader ? atomicAdd(ctr + q, 1u) + per_queue : 0u; }
  // The item of index j of this queue: chunks of consecutive items, dealt to the queues in turn.
  __device__ int item_of(uint32_t j) const {
    const uint32_t c = j / kQueueChunk;
    return (int)((c * (uint32_t)nq + (uint32_t)q) * kQueueChunk + j % kQueueChunk);
  }
  // Called once by each of the launch's `workers` after its last request; the last one resets.
  __device__ void finish(bool leader, uint32_t workers) const {
    if (leader && atomicAdd(ctr + 8, 1u) == workers - 1) {
      for (int i = 0; i < 9; ++i) atomicExch(ctr + i, 0u);
    }
  }
};

template <int DT, int D>
__global__ __launch_bounds__(kDecodeThreads) void prefill_kernel(const PrefillArgs a) {
  extern __shared__ int32_t s_prefix[];  // [num_seqs + 1]: first work item of each sequence
  __shared__ int32_t s_wsum[kWavesPerGroup];
  constexpr int NC = PrefillCfg<DT, D>::kNC;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int qb_queries = NC * (kHeadsPerTile / a.gh_max);
  const int H = a.num_kv_heads * a.n_hg;

  const int total = build_item_prefix(a, qb_queries, s_prefix, s_wsum);

  // The workgroup takes chunks of kQueueChunk (= its four wavefronts) consecutive items from its
  // XCD's queue, one item per wavefront: neighbouring query blocks of one (sequence, kv head),
  // which stream the same K/V pages on one CU. The next chunk is requested while this one runs;
  // its index goes through LDS, double-buffered so that one barrier per chunk suffices.
  static_assert(kQueueChunk == kWavesPerGroup, "one item of a chunk per wavefront");
  __shared__ uint32_t s_next[2];
  const WorkQueue wq(a);
  const bool leader = tid == 0;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t j = wq.rank;
  for (int k = 0;; ++k) {
    const int first = wq.item_of(kQueueChunk * j);
    if (first >= total) break;
    const uint32_t jv = wq.request(leader);
    const int item = first + wv;
    if (item < total) {
      int lo = 0, hi = a.num_seqs;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_prefix[mid] <= item) lo = mid; else hi = mid;
      }
      const int s = lo;
      const int local = item - s_prefix[s];
      // Within a sequence, the query blocks of one (kv head, head group) are consecutive items,
      // so neighbouring waves stream the same K/V pages at about the same time. Later query
      // blocks (longer key ranges) come first.
      const int nqb = (s_prefix[s + 1] - s_prefix[s]) / H;
      const int r = local / nqb;
      const int qb = nqb - 1 - (local - r * nqb);
      prefill_item<DT, D>(a, s, r / a.n_hg, r % a.n_hg, qb, lane);
    }
    // Slot k & 1 was last read in chunk k - 1, before the previous barrier.
    if (leader) s_next[k & 1] = jv;
    __syncthreads();
    j = __builtin_amdgcn_readfirstlane(s_next[k & 1]);
  }
  wq.finish(leader, gridDim.x);
}

// ---------------------------------------------------------------------------------------------
// Workgroup-shared variant (16-bit inputs, head_dim 128). The four wavefronts of a workgroup take four
// consecutive query blocks of one (sequence, kv head, head group), so they need the same keys.
// Each 32-key step is loaded once per workgroup: wavefront 0 loads K of the step's first tile,
// 1 K of the second, 2 and 3 the V tiles; they store them to LDS (double-buffered, one barrier
// per step) and every wavefront reads its matrix-core operands from there. Per step that is a
// quarter of the K/V traffic from L2 of the per-wavefront kernel, which at head_dim 128 is
// bound by exactly that traffic.
//
// LDS buffer of one step (T = one 16-key tile of K or V, 16 * D * 2 bytes), each tile stored
// by its loader as 16-byte chunks in lane order, (j * 64 + lane) * 16 (contiguous, no bank
// conflicts):
//   [0, T)     K tile A: chunk j of lane (kq, ln) = key chunk 4j + kq of token ln, which is
//              exactly the first product's operand, read back by the same lane
//   [T, 2T)    K tile B
//   [2T, 4T)   V of both tiles: the 8 bytes of keys 4kq .. 4kq+3 of dim 32w + e of tile h at
//              (w * 4 + kq) * 512 + (e / 16) * 256 + h * 128 + (e % 16) * 8. A V loader lane's
//              chunk (dims 2ln, 2ln + 1 of one tile) is 16 contiguous bytes there, and eight lanes
//              fill 128 contiguous bytes (no bank conflicts). The second product's operand for dim
//              32w + e and lane group kq is tile A's 8 bytes and tile B's, 128 bytes apart: one
//              paired read, in operand order; lanes ln = 0..15 read 128 contiguous bytes each.
template <int DT, int D>
struct SharedCfg {
  using C = Cfg<DT, D>;
  static constexpr int kNC = prefill_col_tiles(DT, D);
  static constexpr int kTileBytes = kTile * D * C::kE;
  static constexpr int kBufBytes = 4 * kTileBytes;
};

// Offset of key group kq's block in the V layout of one step (chunk / dim group 0).
__device__ __forceinline__ int j0_kq_base(int kq) { return kq * 512; }

template <int DT, int D>
__device__ __forceinline__ void prefill_shared_item(const PrefillArgs& a, int s, int g, int hg, int qbg, int wv,
                                                    int lane, char* lds) {
  using C = Cfg<DT, D>;
  using SC = SharedCfg<DT, D>;
  static_assert(DT != kF32, "the shared variant takes 16-bit inputs");
  constexpr int NC = SC::kNC;
  constexpr int T = SC::kTileBytes;
  const int kq = lane >> 4;
  const int ln = lane & 15;
  const int bs = a.block_size;
  int L, q0, n;
  seq_rows(a, s, L, q0, n);
  const int gh = a.gh_max;
  const int qpt = kHeadsPerTile / gh;
  const int qb_queries = NC * qpt;
  // The workgroup's queries and keys (the same in every wavefront).
  const int wg_first = qbg * kWavesPerGroup * qb_queries;
  const int wg_last = min(n, wg_first + kWavesPerGroup * qb_queries) - 1;
  const int p_last_wg = L - n + wg_last;
  // This wavefront's query block; a workgroup at the end of a sequence may have idle wavefronts,
  // which still load their share and meet every barrier.
  const int qfirst = wg_first + wv * qb_queries;
  const bool active = qfirst < n;
  const int p_first = L - n + qfirst;

  int qi[NC], hh[NC], pos[NC];
  bool valid[NC];
#pragma unroll
  for (int ct = 0; ct < NC; ++ct) {
    const int ql = ln / gh;
    const int hl = hg * kHeadsPerTile + (ln % gh);
    qi[ct] = qfirst + ct * qpt + ql;
    hh[ct] = g * a.group + hl;
    valid[ct] = active && ql < qpt && hl < a.group && qi[ct] < n;
    pos[ct] = valid[ct] ? L - n + qi[ct] : p_last_wg;
  }
  const uint32_t qflip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  const float c = fmaxf(fabsf(a.scale_log2), FLT_MIN);
  u4 qv[NC][C::kLoads];
#pragma unroll
  for (int ct = 0; ct < NC; ++ct) {
    const char* qrow = reinterpret_cast<const char*>(a.q) +
                       ((int64_t)(q0 + qi[ct]) * a.q_token_stride + (int64_t)hh[ct] * D) * C::kE;
#pragma unroll
    for (int j = 0; j < C::kLoads; ++j) {
      qv[ct][j] = valid[ct] ? *reinterpret_cast<const u4*>(qrow + (4 * j + kq) * 16) : u4{0u, 0u, 0u, 0u};
      qv[ct][j] ^= u4{qflip, qflip, qflip, qflip};
    }
  }
  f4 acc[NC][C::kAcc];
  f4 accl[NC];  // fp16: running sums of the rounded weights (matrix cores; every row the same)
  float m[NC], l[NC];
  float thr[NC];  // (m + 8) / c: a raw score above it moves the running maximum
#pragma unroll
  for (int ct = 0; ct < NC; ++ct) {
    m[ct] = -INFINITY;
    thr[ct] = -INFINITY;
    l[ct] = 0.f;
#pragma unroll
    for (int u = 0; u < C::kAcc; ++u) acc[ct][u] = f4{0.f, 0.f, 0.f, 0.f};
    accl[ct] = f4{0.f, 0.f, 0.f, 0.f};
  }
  // Matrix-core weight sums (fp16): an all-ones operand, kept in registers.
  u4 ones_u = u4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
  asm volatile("" : "+v"(ones_u));
  const h8 ones8 = __builtin_bit_cast(h8, ones_u);
  (void)ones8;

  const int64_t page_bytes = (int64_t)bs * D * C::kE;
  const int page_bytes32 = (int)page_bytes;
  const int64_t blk_stride = (int64_t)a.num_kv_heads * page_bytes;
  const int nb_max = (int)(a.num_blocks - 1 < INT32_MAX ? a.num_blocks - 1 : INT32_MAX);
  const int tiles = p_last_wg / kTile + 1;
  const int steps = (tiles + 1) >> 1;
  const_i32* cbt = (const_i32*)(a.block_tables + (int64_t)s * a.max_blocks);

  // This wavefront's share of each step: K (wv < 2) or V (wv >= 2) of tile A (even wv) or B.
  // The same instructions for every share (the base and lane offsets are selected), so each
  // wavefront's loads are unconditional and the compiler's wait counts stay exact.
  const bool share_k = wv < 2;
  const int half = wv & 1;
  const char* sbase = reinterpret_cast<const char*>(share_k ? a.k_cache : a.v_cache) + (int64_t)g * page_bytes;
  // K: chunk (4j + kq) of token (off0 + ln); V: tokens off0 + 4kq .. +3 of dims 32j + 2ln, +1.
  const int lane_off = share_k ? (kq * bs + ln) * 16 : (kq * D + 2 * ln) * 8;
  const int j_stride = share_k ? 64 * bs : 256;
  const int off_per_key = share_k ? 16 : D * C::kE;
  auto share_tile = [&](int st) { return min(2 * st + half, tiles - 1); };
  u4 stg[C::kLoads];
  auto load_share = [&](int st, int raw) {
    const int tile = share_tile(st);
    const int64_t blk = min(max((int)__builtin_amdgcn_readfirstlane(raw), 0), nb_max);
    // A tile that does not exist (an odd last step) loads zeros and reads no memory.
    const int bytes = 2 * st + half < tiles ? page_bytes32 : 0;
    const __amdgpu_buffer_rsrc_t r = page_rsrc(sbase + blk * blk_stride, bytes);
    const int off = lane_off + ((tile * kTile) & (bs - 1)) * off_per_key;
#pragma unroll
    for (int j = 0; j < C::kLoads; ++j) stg[j] = buf_load16<kPolicyDefault>(r, off + j * j_stride);
  };
  auto bt_entry = [&](int st) -> int {
    return cbt[(share_tile(min(st, steps - 1)) * kTile) >> a.bs_log2];
  };
  // Values of keys at or beyond L may be anything: zero them before they are shared.
  auto store_share = [&](int st, char* buf) {
    if (!share_k) {
      const int t0 = share_tile(st) * kTile;
      // Only a sequence's last tile reaches past L: kept a real, wave-uniform branch.
      const int past = __builtin_amdgcn_readfirstlane(t0 + kTile > L ? 1 : 0);
      if (__builtin_expect(past != 0, 0)) {
        const bool v0 = t0 + 4 * kq + 0 < L, v1 = t0 + 4 * kq + 1 < L;
        const bool v2 = t0 + 4 * kq + 2 < L, v3 = t0 + 4 * kq + 3 < L;
        const uint32_t m01 = (v0 ? 0x0000FFFFu : 0u) | (v1 ? 0xFFFF0000u : 0u);
        const uint32_t m23 = (v2 ? 0x0000FFFFu : 0u) | (v3 ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int j = 0; j < C::kLoads; ++j) stg[j] &= u4{m01, m23, m01, m23};
      }
    }
    if (share_k) {
      char* dst = buf + wv * T + lane * 16;
#pragma unroll
      for (int j = 0; j < C::kLoads; ++j) *reinterpret_cast<u4*>(dst + j * 1024) = stg[j];
    } else {
      // V: the chunk (dims 32j + 2ln, +1 of key group kq) is 16 contiguous bytes of the layout
      // below; eight lanes fill 128 contiguous bytes.
      char* dst = buf + 2 * T + (j0_kq_base(kq) + (ln >> 3) * 256 + half * 128 + (ln & 7) * 16);
#pragma unroll
      for (int j = 0; j < C::kLoads; ++j) *reinterpret_cast<u4*>(dst + j * 2048) = stg[j];
    }
  };


  int raw_next = bt_entry(1);
  load_share(0, bt_entry(0));
  store_share(0, lds);
  __syncthreads();
  for (int st = 0; st < steps; ++st) {
    char* buf = lds + (st & 1) * SC::kBufBytes;
    // Next step's share: in flight during this step's arithmetic (re-reads the last step at the end).
    load_share(st + 1, raw_next);
    __builtin_amdgcn_sched_barrier(0);
    raw_next = bt_entry(st + 2);

    if (active) {
      const int t0 = st * 2 * kTile;
      u4 kA[C::kLoads], kB[C::kLoads];
#pragma unroll
      for (int j = 0; j < C::kLoads; ++j) {
        kA[j] = *reinterpret_cast<const u4*>(buf + (j * 64 + lane) * 16);
        kB[j] = *reinterpret_cast<const u4*>(buf + T + (j * 64 + lane) * 16);
      }
      f4 sA[NC], sB[NC];
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        sA[ct] = f4{0.f, 0.f, 0.f, 0.f};
        sB[ct] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < C::kLoads; ++j) {
          if constexpr (DT == kBF16) {
            sA[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, kA[j]),
                                                             __builtin_bit_cast(b8, qv[ct][j]), sA[ct], 0, 0, 0);
            sB[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, kB[j]),
                                                             __builtin_bit_cast(b8, qv[ct][j]), sB[ct], 0, 0, 0);
          } else {
            sA[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, kA[j]),
                                                            __builtin_bit_cast(h8, qv[ct][j]), sA[ct], 0, 0, 0);
            sB[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, kB[j]),
                                                            __builtin_bit_cast(h8, qv[ct][j]), sB[ct], 0, 0, 0);
          }
        }
      }
      // V^T operands: dims 32w + ln (va0) and 32w + 16 + ln (va1), keys of tile A then tile B:
      // each two 8-byte reads 128 bytes apart (one paired LDS read), in operand order.
      u4 va0[C::kLoads], va1[C::kLoads];
#pragma unroll
      for (int w = 0; w < C::kLoads; ++w) {
        const char* va = buf + 2 * T + w * 2048 + j0_kq_base(kq) + ln * 8;
        const u2 a0 = *reinterpret_cast<const u2*>(va), b0 = *reinterpret_cast<const u2*>(va + 128);
        const u2 a1 = *reinterpret_cast<const u2*>(va + 256), b1 = *reinterpret_cast<const u2*>(va + 384);
        va0[w] = u4{a0[0], a0[1], b0[0], b0[1]};
        va1[w] = u4{a1[0], a1[1], b1[0], b1[1]};
      }
      const bool open = t0 + 2 * kTile - 1 <= p_first;
      // One causal-mask branch and one rescale branch for all column tiles, as in prefill_item.
      float x[NC][8];
#pragma unroll
      for (int ct = 0; ct < NC; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[ct][r] = sA[ct][r];
          x[ct][4 + r] = sB[ct][r];
        }
      if (!open) {
#pragma unroll
        for (int ct = 0; ct < NC; ++ct)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int t = t0 + (j < 4 ? 0 : kTile) + 4 * kq + (j & 3);
            if (t > pos[ct]) x[ct][j] = -INFINITY;
          }
      }
      // The running maximum moves only on jumps above 8; each lane tests its own scores, and the
      // maximum over a column's rows is taken only when some lane finds a jump (as in prefill_item).
      float alpha[NC];
      bool jump = false;
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        alpha[ct] = 1.0f;
        jump = jump | (fmax8(x[ct]) > thr[ct]);
      }
      if (__builtin_amdgcn_ballot_w64(jump) != 0) {
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
          const float mt = max_over_rows(fmax8(x[ct]));
          const float m_cand = __builtin_elementwise_maximum(m[ct], mt * c);
          const float m_use = m_cand > m[ct] + 8.0f ? m_cand : m[ct];
          alpha[ct] = exp2_fast(m[ct] - m_use);
          m[ct] = m_use;
          thr[ct] = (m_use + 8.0f) / c;
#pragma unroll
          for (int u = 0; u < C::kAcc; ++u) acc[ct][u] *= alpha[ct];
          accl[ct] *= alpha[ct];
        }
      }
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = exp2_fast(fmaf(x[ct][j], c, weight_log2_scale<DT>(8) - m[ct]));
        // fp16: the running sum is taken over the rounded weights, on the matrix cores (below)
        if constexpr (DT != kF16)
          l[ct] = fmaf(l[ct], alpha[ct], ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
        u4 ph, pl;  // pl: bf16 remainder parts
        if constexpr (DT == kBF16) {
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) {
            const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{p[2 * i2], p[2 * i2 + 1]}, bf2));
            const float r0 = p[2 * i2] - __uint_as_float(hb << 16);
            const float r1 = p[2 * i2 + 1] - __uint_as_float(hb & 0xFFFF0000u);
            ph[i2] = hb;
            pl[i2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{r0, r1}, bf2));
          }
        } else {
          // fp16: one part, rounded to nearest (relative error <= 2^-11). The running sum is of
          // exactly these rounded weights, taken on the matrix cores (an all-ones row operand:
          // every output row is the column's sum over the 32 keys, in fp32), so the
          // normalisation matches the product: equal weights, or one dominant weight, give their
          // values' mean exactly.
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2)
            ph[i2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{p[2 * i2], p[2 * i2 + 1]}, hf2));
          accl[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones8, __builtin_bit_cast(h8, ph), accl[ct], 0, 0, 0);
        }
#pragma unroll
        for (int w = 0; w < C::kLoads; ++w) {
          if constexpr (DT == kBF16) {
            const b8 bh = __builtin_bit_cast(b8, ph), bl = __builtin_bit_cast(b8, pl);
            const b8 a0 = __builtin_bit_cast(b8, va0[w]), a1 = __builtin_bit_cast(b8, va1[w]);
            acc[ct][2 * w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bh, acc[ct][2 * w], 0, 0, 0);
            acc[ct][2 * w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bl, acc[ct][2 * w], 0, 0, 0);
            acc[ct][2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bh, acc[ct][2 * w + 1], 0, 0, 0);
            acc[ct][2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bl, acc[ct][2 * w + 1], 0, 0, 0);
          } else {
            const h8 hh8 = __builtin_bit_cast(h8, ph);
            const h8 a0 = __builtin_bit_cast(h8, va0[w]), a1 = __builtin_bit_cast(h8, va1[w]);
            acc[ct][2 * w] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, hh8, acc[ct][2 * w], 0, 0, 0);
            acc[ct][2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, hh8, acc[ct][2 * w + 1], 0, 0, 0);
          }
        }
      }
    }
    // The other buffer was last read in the previous step, before its barrier.
    store_share(st + 1, lds + ((st + 1) & 1) * SC::kBufBytes);
    __syncthreads();
  }

  if (!active) return;
#pragma unroll
  for (int ct = 0; ct < NC; ++ct) {
    float lt;
    if constexpr (DT == kF16) {
      lt = accl[ct][0];  // already summed over all keys (and lane groups) by the matrix cores
    } else {
      lt = l[ct] + __shfl_xor(l[ct], 16);
      lt += __shfl_xor(lt, 32);
    }
    const float inv = 1.0f / lt;
    if (!valid[ct]) continue;
    const int64_t base = ((int64_t)(q0 + qi[ct]) * a.num_heads + hh[ct]) * D;
#pragma unroll
    for (int w = 0; w < C::kLoads; ++w) {
      const float v0[4] = {acc[ct][2 * w][0] * inv, acc[ct][2 * w][1] * inv, acc[ct][2 * w][2] * inv,
                           acc[ct][2 * w][3] * inv};
      const float v1[4] = {acc[ct][2 * w + 1][0] * inv, acc[ct][2 * w + 1][1] * inv, acc[ct][2 * w + 1][2] * inv,
                           acc[ct][2 * w + 1][3] * inv};
      store4<DT>(a.out, base + 32 * w + 4 * kq, v0, a.out_f32 != 0);
      store4<DT>(a.out, base + 32 * w + 16 + 4 * kq, v1, a.out_f32 != 0);
    }
  }
}

// Workgroup-level items: (sequence, kv head, head group, group of four query blocks), on
// persistent workgroups. Dynamic LDS: the item prefix ([num_seqs + 1] ints, rounded up to 16
// bytes), then two step buffers.
template <int DT, int D>
__global__ __launch_bounds__(kDecodeThreads) void prefill_shared_kernel(const PrefillArgs a) {
  extern __shared__ __align__(16) int32_t s_dyn[];
  __shared__ int32_t s_wsum[kWavesPerGroup];
  __shared__ uint32_t s_next;
  constexpr int NC = SharedCfg<DT, D>::kNC;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg_queries = kWavesPerGroup * NC * (kHeadsPerTile / a.gh_max);
  const int H = a.num_kv_heads * a.n_hg;
  int32_t* s_prefix = s_dyn;
  char* bufs = reinterpret_cast<char*>(s_dyn + ((a.num_seqs + 1 + 3) & ~3));
  const int total = build_item_prefix(a, wg_queries, s_prefix, s_wsum);
  // Items from this XCD's queue: thread 0 requests the next index while the current item runs
  // and leaves it in LDS before the item's last barrier.
  const WorkQueue wq(a);
  const bool leader = tid == 0;
  if (leader) s_next = wq.rank;
  __syncthreads();
  for (;;) {
    const int item = wq.item_of((uint32_t)__builtin_amdgcn_readfirstlane(s_next));
    if (item >= total) break;
    const uint32_t jv = wq.request(leader);
    int lo = 0, hi = a.num_seqs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_prefix[mid] <= item) lo = mid; else hi = mid;
    }
    const int s = __builtin_amdgcn_readfirstlane(lo);
    const int local = item - s_prefix[s];
    const int nqb = (s_prefix[s + 1] - s_prefix[s]) / H;
    const int r = local / nqb;
    const int qbg = __builtin_amdgcn_readfirstlane(nqb - 1 - (local - r * nqb));
    const int rr = __builtin_amdgcn_readfirstlane(r);
    prefill_shared_item<DT, D>(a, s, rr / a.n_hg, rr % a.n_hg, qbg, wv, lane, bufs);
    // Every wavefront has read s_next (above); the barrier after this store publishes the next
    // index, and the next item's first store goes to buffer 0, which this item may have read last.
    if (leader) s_next = jv;
    __syncthreads();
  }
  wq.finish(leader, gridDim.x);
}

template <int DT, int D>
hipError_t launch_prefill_shared_t(const PrefillArgs& a, int grid, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((prefill_shared_kernel<DT, D>), dim3(grid), dim3(kDecodeThreads), lds, st, a);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_prefill_t(const PrefillArgs& a, int grid, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((prefill_kernel<DT, D>), dim3(grid), dim3(kDecodeThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace

int prefill_queries_per_item(int dtype, int head_dim, int gh_max) {
  return prefill_col_tiles(dtype, head_dim) * (kHeadsPerTile / gh_max);
}

size_t prefill_shared_buffer_bytes(int head_dim) {
  return head_dim == 128 ? 2 * (size_t)SharedCfg<kBF16, 128>::kBufBytes : 0;
}

hipError_t launch_prefill_shared(const PrefillArgs& a, int dtype, int head_dim, int grid, size_t lds,
                                 hipStream_t st) {
  if (head_dim != 128) return hipErrorInvalidValue;
  if (dtype == kF16) return launch_prefill_shared_t<kF16, 128>(a, grid, lds, st);
  if (dtype == kBF16) return launch_prefill_shared_t<kBF16, 128>(a, grid, lds, st);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int grid, size_t lds, hipStream_t st) {
  switch (dtype) {
    case kF32:
      if (head_dim == 64) return launch_prefill_t<kF32, 64>(a, grid, lds, st);
      if (head_dim == 128) return launch_prefill_t<kF32, 128>(a, grid, lds, st);
      if (head_dim == 256) return launch_prefill_t<kF32, 256>(a, grid, lds, st);
      break;
    case kF16:
      if (head_dim == 64) return launch_prefill_t<kF16, 64>(a, grid, lds, st);
      if (head_dim == 128) return launch_prefill_t<kF16, 128>(a, grid, lds, st);
      if (head_dim == 256) return launch_prefill_t<kF16, 256>(a, grid, lds, st);
      break;
    case kBF16:
      if (head_dim == 64) return launch_prefill_t<kBF16, 64>(a, grid, lds, st);
      if (head_dim == 128) return launch_prefill_t<kBF16, 128>(a, grid, lds, st);
      if (head_dim == 256) return launch_prefill_t<kBF16, 256>(a, grid, lds, st);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
