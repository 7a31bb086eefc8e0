// KV-cache scatter for gfx950: each decode step's new K/V rows are copied into
// their cache slots (miniVLLM documentation, "What is miniVLLM?": paged KV
// cache management). Bit copies, no conversion.
//
// One thread per (token, kv head, 16-byte chunk of the row). The K chunk maps
// to one 16-byte run of the K page (layout [.. D/x][bs][x]). Each thread also
// moves x value elements of the token to x dims of the V page (layout
// [.. bs/4][D][4]), each at the token's position inside its group of four.

#include "pa_internal.h"

#include <type_traits>

namespace pa {
namespace {

typedef unsigned int u4 __attribute__((ext_vector_type(4)));

template <int E>
__global__ __launch_bounds__(256) void store_kernel(const StoreArgs a) {
  constexpr int kX = 16 / E;  // elements per 16-byte chunk
  const int chunks = a.head_dim / kX;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = (int64_t)a.num_kv_heads * chunks;
  if (idx >= (int64_t)a.num_tokens * per_token) return;
  const int i = (int)(idx / per_token);
  const int rem = (int)(idx - (int64_t)i * per_token);
  const int g = rem / chunks;
  const int c = rem - g * chunks;
  const int64_t slot = a.slot_mapping[i];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot / a.block_size;
  const int o = (int)(slot - blk * a.block_size);
  const int64_t page = (blk * a.num_kv_heads + g) * (int64_t)a.block_size * a.head_dim;  // elements

  const char* ksrc = reinterpret_cast<const char*>(a.k) + ((int64_t)i * a.k_stride + (int64_t)g * a.head_dim + (int64_t)c * kX) * E;
  const u4 kv = *reinterpret_cast<const u4*>(ksrc);
  // V: in step j, lane c of a (token, head) takes dim j * chunks + c. The lanes of one store
  // then write neighbouring dims, 4 * E bytes apart in the page, and those writes combine into
  // a few memory requests (with dims c * kX + j each lane's writes would fall in a segment of
  // its own). Loads first, so that they are in flight together.
  using VE = typename std::conditional<E == 4, uint32_t, uint16_t>::type;
  const VE* vsrc = reinterpret_cast<const VE*>(reinterpret_cast<const char*>(a.v) +
                                               ((int64_t)i * a.v_stride + (int64_t)g * a.head_dim) * E);
  VE vv[kX];
#pragma unroll
  for (int j = 0; j < kX; ++j) vv[j] = vsrc[j * chunks + c];

  char* kdst = reinterpret_cast<char*>(a.k_cache) + (page + ((int64_t)c * a.block_size + o) * kX) * E;
  *reinterpret_cast<u4*>(kdst) = kv;

  // V element (o, d) sits at [(o / 4) * D + d] * 4 + o % 4 within the page.
  VE* vdst = reinterpret_cast<VE*>(reinterpret_cast<char*>(a.v_cache) + page * E);
  const int64_t vrow = (int64_t)(o >> 2) * a.head_dim * 4 + (o & 3);
#pragma unroll
  for (int j = 0; j < kX; ++j) vdst[vrow + (int64_t)(j * chunks + c) * 4] = vv[j];
}

// Whole-block copies for copy-on-write: one thread per (pair, 16-byte chunk of a block's
// K or V region); a block is num_kv_heads contiguous pages in each cache.
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* k_cache, char* v_cache, const int32_t* src,
                                                          const int32_t* dst, int32_t num_pairs, int64_t block_bytes,
                                                          int64_t num_blocks) {
  const int64_t chunks = block_bytes / 16;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)num_pairs * chunks * 2) return;
  const int64_t pair = idx / (chunks * 2);
  const int64_t rem = idx - pair * chunks * 2;
  const bool is_v = rem >= chunks;
  const int64_t c = is_v ? rem - chunks : rem;
  const int64_t s = src[pair], d = dst[pair];
  if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) return;
  char* base = is_v ? v_cache : k_cache;
  const u4 v = *reinterpret_cast<const u4*>(base + s * block_bytes + c * 16);
  *reinterpret_cast<u4*>(base + d * block_bytes + c * 16) = v;
}

}  // namespace

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst,
                              int32_t num_pairs, int64_t block_bytes, int64_t num_blocks, hipStream_t st) {
  const int64_t threads = (int64_t)num_pairs * (block_bytes / 16) * 2;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<char*>(k_cache), reinterpret_cast<char*>(v_cache), src, dst, num_pairs,
                     block_bytes, num_blocks);
  return hipGetLastError();
}

hipError_t launch_store(const StoreArgs& a, int dtype, hipStream_t st) {
  const int e = elem_bytes(dtype);
  const int64_t threads = (int64_t)a.num_tokens * a.num_kv_heads * (a.head_dim / (16 / e));
  if (threads == 0) return hipSuccess;
  const int64_t grid = (threads + 255) / 256;
  if (e == 4)
    hipLaunchKernelGGL(store_kernel<4>, dim3((unsigned)grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(store_kernel<2>, dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pa
