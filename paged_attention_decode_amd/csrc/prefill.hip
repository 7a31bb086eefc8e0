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
// streams the sequence's 16-token K/V tiles up to the block's last query and
// keeps, per column, an online-softmax state. The 16 columns of a matrix-core
// tile are (query, head) pairs: 16/G queries x G heads of one kv head (or 16
// heads of one query when G > 16). Several column tiles share each K/V load:
// four at head_dim 64, two at 128, one at 256. Per tile:
//   S[t][c]   = K[t][:] . Q[c][:]           (rows = tokens, cols = (query, head))
//   causal mask per column, online softmax per column
//   O^T[d][c] += V^T[d][t] . P^T[t][c]      (P as a sum of two 16-bit parts)
// The operand layouts are those of the decode kernel (same cache layout). K/V
// tiles are reused by every query block of the sequence, so they are loaded
// with the default (caching) policy.

#include "device_common.h"

namespace pa {
namespace {

using namespace dev;

#ifndef PA_PREFILL_NC64
#define PA_PREFILL_NC64 4
#endif

// Column tiles per wavefront: every K/V tile loaded serves 16 * kNC columns.
constexpr int prefill_col_tiles(int head_dim) { return head_dim <= 64 ? PA_PREFILL_NC64 : (head_dim <= 128 ? 2 : 1); }

template <int DT, int D>
struct PrefillCfg {
  using C = Cfg<DT, D>;
  static constexpr int kNC = prefill_col_tiles(D);
};

template <int DT, int D>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, int s, int g, int hg, int qb, int lane) {
  using C = Cfg<DT, D>;
  constexpr int NC = PrefillCfg<DT, D>::kNC;
  const int kq = lane >> 4;
  const int ln = lane & 15;
  const int bs = a.block_size;
  const int max_len = a.max_blocks << a.bs_log2;
  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > max_len ? max_len : L);
  const int q0 = a.query_start[s];
  int n = a.query_start[s + 1] - q0;
  n = n < 0 ? 0 : (n > L ? L : n);
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
  u4 qv[NC][C::kLoads];
#pragma unroll
  for (int ct = 0; ct < NC; ++ct) {
    const char* qrow = reinterpret_cast<const char*>(a.q) +
                       ((int64_t)(q0 + qi[ct]) * a.q_token_stride + (int64_t)hh[ct] * D) * C::kE;
#pragma unroll
    for (int j = 0; j < C::kLoads; ++j)
      qv[ct][j] = valid[ct] ? *reinterpret_cast<const u4*>(qrow + (4 * j + kq) * 16) : u4{0u, 0u, 0u, 0u};
  }

  f4 acc[NC][C::kAcc];
  float m[NC], l[NC];
#pragma unroll
  for (int ct = 0; ct < NC; ++ct) {
    m[ct] = -INFINITY;
    l[ct] = 0.f;
#pragma unroll
    for (int u = 0; u < C::kAcc; ++u) acc[ct][u] = f4{0.f, 0.f, 0.f, 0.f};
  }

  const int64_t page_bytes = (int64_t)bs * D * C::kE;
  const int page_bytes32 = (int)page_bytes;
  const int64_t blk_stride = (int64_t)a.num_kv_heads * page_bytes;
  const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (int64_t)g * page_bytes;
  const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (int64_t)g * page_bytes;
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;
  const int64_t nb_max = a.num_blocks - 1;
  const uint32_t k_lane = (uint32_t)((kq * bs + ln) * 16);
  const uint32_t v_lane = (DT == kF32) ? (uint32_t)((kq * D + ln) * 16) : (uint32_t)((kq * D + 2 * ln) * 8);
  int bt_first = INT32_MIN / 2;
  int bt_val = 0;

  auto load_tile = [&](int i, u4 (&kb)[C::kLoads], u4 (&vb)[C::kLoads]) {
    const int t0 = i * kTile;
    const int page = t0 >> a.bs_log2;
    const int off0 = t0 & (bs - 1);
    if (page - bt_first >= 64 || page < bt_first) {
      bt_first = page;
      const int idx = page + lane;
      bt_val = idx < a.max_blocks ? bt[idx] : 0;
    }
    int64_t blk = __builtin_amdgcn_readlane(bt_val, page - bt_first);
    blk = blk < 0 ? 0 : (blk > nb_max ? nb_max : blk);
    const __amdgpu_buffer_rsrc_t kr = page_rsrc(kbase + blk * blk_stride, page_bytes32);
    const __amdgpu_buffer_rsrc_t vr = page_rsrc(vbase + blk * blk_stride, page_bytes32);
    const int koff = (int)k_lane + off0 * 16;
    const int voff = (int)v_lane + off0 * D * C::kE;
#pragma unroll
    for (int j = 0; j < C::kLoads; ++j) kb[j] = buf_load16<kPolicyDefault>(kr, koff + j * 64 * bs);
#pragma unroll
    for (int j = 0; j < C::kLoads; ++j) vb[j] = buf_load16<kPolicyDefault>(vr, voff + j * 256);
  };

  auto compute_tile = [&](int i, const u4 (&kb)[C::kLoads], u4 (&vb)[C::kLoads]) {
    const int t0 = i * kTile;
    const bool open = t0 + kTile - 1 <= p_first;  // every key of the tile visible to every column
    const bool past_end = t0 + kTile > L;
    if (past_end) {
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
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
      f4 sv = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < C::kLoads; ++j) {
        if constexpr (DT == kF32) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sv = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kb[j][e]), __uint_as_float(qv[ct][j][e]), sv,
                                                      0, 0, 0);
        } else if constexpr (DT == kBF16) {
          sv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, kb[j]), __builtin_bit_cast(b8, qv[ct][j]),
                                                       sv, 0, 0, 0);
        } else {
          sv = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, kb[j]), __builtin_bit_cast(h8, qv[ct][j]),
                                                      sv, 0, 0, 0);
        }
      }
      float z[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[r] = sv[r] * a.scale_log2;
        const int t = t0 + 4 * kq + r;
        if (!open && (t > pos[ct] || t >= L)) z[r] = -INFINITY;
      }
      float mt = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m[ct], mt);
      const float alpha = exp2_fast(m[ct] - m_new);
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = exp2_fast(z[r] - m_new);
      l[ct] = l[ct] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
      m[ct] = m_new;
#pragma unroll
      for (int u = 0; u < C::kAcc; ++u) acc[ct][u] *= alpha;
      if constexpr (DT == kF32) {
#pragma unroll
        for (int u = 0; u < C::kLoads; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[ct][u] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vb[u][e]), p[e], acc[ct][u], 0, 0, 0);
      } else if constexpr (DT == kBF16) {
        s4 ph, pl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t hb = bf16_bits_rne(p[r]);
          ph[r] = (short)hb;
          pl[r] = (short)bf16_bits_rne(p[r] - __uint_as_float(hb << 16));
        }
#pragma unroll
        for (int w = 0; w < C::kLoads; ++w) {
          const s4 a0 = __builtin_bit_cast(s4, u2{vb[w].x, vb[w].y});
          const s4 a1 = __builtin_bit_cast(s4, u2{vb[w].z, vb[w].w});
          acc[ct][2 * w] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a0, ph, acc[ct][2 * w], 0, 0, 0);
          acc[ct][2 * w] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a0, pl, acc[ct][2 * w], 0, 0, 0);
          acc[ct][2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a1, ph, acc[ct][2 * w + 1], 0, 0, 0);
          acc[ct][2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a1, pl, acc[ct][2 * w + 1], 0, 0, 0);
        }
      } else {
        h4 ph, pl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const _Float16 hi = (_Float16)p[r];
          ph[r] = hi;
          pl[r] = (_Float16)(p[r] - (float)hi);
        }
#pragma unroll
        for (int w = 0; w < C::kLoads; ++w) {
          const h4 a0 = __builtin_bit_cast(h4, u2{vb[w].x, vb[w].y});
          const h4 a1 = __builtin_bit_cast(h4, u2{vb[w].z, vb[w].w});
          acc[ct][2 * w] = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, ph, acc[ct][2 * w], 0, 0, 0);
          acc[ct][2 * w] = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, pl, acc[ct][2 * w], 0, 0, 0);
          acc[ct][2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, ph, acc[ct][2 * w + 1], 0, 0, 0);
          acc[ct][2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, pl, acc[ct][2 * w + 1], 0, 0, 0);
        }
      }
    }
  };

  // Keys 0 .. p_last; the loads of tile i+1 are in flight while tile i is computed.
  const int tiles = p_last / kTile + 1;
  u4 kA[C::kLoads], vA[C::kLoads], kB[C::kLoads], vB[C::kLoads];
  int i = 0;
  load_tile(i, kA, vA);
  while (true) {
    const bool has_b = i + 1 < tiles;
    if (has_b) load_tile(i + 1, kB, vB);
    compute_tile(i, kA, vA);
    if (!has_b) break;
    const bool has_a = i + 2 < tiles;
    if (has_a) load_tile(i + 2, kA, vA);
    compute_tile(i + 1, kB, vB);
    if (!has_a) break;
    i += 2;
  }

#pragma unroll
  for (int ct = 0; ct < NC; ++ct) {
    float lt = l[ct] + __shfl_xor(l[ct], 16);
    lt += __shfl_xor(lt, 32);
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
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = acc[ct][2 * w + (j & 1)][j >> 1] * inv;
        store8<DT>(a.out, base + 32 * w + 8 * kq, v, a.out_f32 != 0);
      }
    }
  }
}

template <int DT, int D>
__global__ __launch_bounds__(kDecodeThreads) void prefill_kernel(const PrefillArgs a) {
  extern __shared__ int32_t s_prefix[];  // [num_seqs + 1]: first work item of each sequence
  __shared__ int32_t s_wsum[kWavesPerGroup];
  constexpr int NC = PrefillCfg<DT, D>::kNC;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Workgroups are dealt round-robin to the 8 XCDs; renumber them so that consecutive
  // waves, which take consecutive items, run on one XCD and share its L2.
  int grp = blockIdx.x;
  if ((gridDim.x & 7) == 0) grp = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int wave = grp * kWavesPerGroup + __builtin_amdgcn_readfirstlane(tid >> 6);
  const int max_len = a.max_blocks << a.bs_log2;
  const int qb_queries = NC * (kHeadsPerTile / a.gh_max);
  const int H = a.num_kv_heads * a.n_hg;

  // Items per sequence: ceil(n / queries per block) * kv heads * head groups.
  int carry = 0;
  for (int base = 0; base < a.num_seqs; base += kDecodeThreads) {
    const int i = base + tid;
    int v = 0;
    if (i < a.num_seqs) {
      int L = a.context_lens[i];
      L = L < 0 ? 0 : (L > max_len ? max_len : L);
      int n = a.query_start[i + 1] - a.query_start[i];
      n = n < 0 ? 0 : (n > L ? L : n);
      v = ((n + qb_queries - 1) / qb_queries) * H;
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

  for (int item = wave; item < total; item += a.num_waves) {
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
}

template <int DT, int D>
hipError_t launch_prefill_t(const PrefillArgs& a, int grid, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((prefill_kernel<DT, D>), dim3(grid), dim3(kDecodeThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace

int prefill_queries_per_item(int head_dim, int gh_max) {
  return prefill_col_tiles(head_dim) * (kHeadsPerTile / gh_max);
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
