// Streaming-read ceiling for the decode benchmark (measurement only; built as its own library,
// libpa_stream_read.so, and not part of libpagedattn's ABI).
//
// Reads a large device buffer once with the loads the decode kernel uses for K/V pages: 16-byte
// buffer loads, every lane of a wavefront on consecutive 16-byte chunks (1 KiB per load
// instruction), with the default or the non-temporal cache policy. Each wavefront keeps UNROLL
// such loads in flight per round and walks the buffer with a stride of all wavefronts' rounds.
// The loaded words are summed into one 32-bit word per lane and written to `sink`, so no
// load is dead; the sink is 256 bytes per wavefront, negligible next to the buffer.
//
// The rate this kernel reaches is the practical HBM read ceiling of the GPU for this access
// pattern: the decode kernel's K/V bandwidth is reported as a fraction of it as well as of the
// 8 TB/s peak.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRsrcWord3 = 0x00020000;

template <int POL, int UNROLL>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* buf, uint32_t bytes, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const uint32_t wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const uint32_t waves = gridDim.x * (kThreads / 64);
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(buf), (short)0, (int)bytes, kRsrcWord3);
  constexpr uint32_t kRound = UNROLL * 1024u;
  const uint64_t stride = (uint64_t)waves * kRound;
  // One round = UNROLL consecutive 1 KiB loads. Two register sets: the next round's loads are
  // issued before this round's are folded, so a wavefront always has loads in flight (as the
  // decode kernel keeps the next tile's loads in flight while it computes one). A round past the
  // end reads from offset `bytes`, which the buffer resource returns as zeros without a memory
  // access.
  auto load = [&](uint64_t c, u4 (&v)[UNROLL]) {
    const uint32_t base = c < bytes ? (uint32_t)c : bytes;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      v[u] = __builtin_bit_cast(
          u4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(base + (c < bytes ? u * 1024u + lane * 16u : 0u)), 0,
                                                    POL));
  };
  u4 acc = u4{0u, 0u, 0u, 0u};
  u4 va[UNROLL], vb[UNROLL];
  uint64_t c = (uint64_t)wave * kRound;
  load(c, va);
  // Each round is folded exactly once; the loop leaves when the round just folded was the last.
  while (true) {
    load(c + stride, vb);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc += va[u];
    c += stride;
    if (c >= bytes) break;
    load(c + stride, va);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc += vb[u];
    c += stride;
    if (c >= bytes) break;
  }
  sink[(uint64_t)wave * 64 + lane] = acc.x + acc.y + acc.z + acc.w;
}

template <int POL>
hipError_t launch_pol(int unroll, const void* buf, uint32_t bytes, int grid, uint32_t* sink, hipStream_t s) {
  const char* b = static_cast<const char*>(buf);
  switch (unroll) {
    case 4: hipLaunchKernelGGL((stream_read_kernel<POL, 4>), dim3(grid), dim3(kThreads), 0, s, b, bytes, sink); break;
    case 8: hipLaunchKernelGGL((stream_read_kernel<POL, 8>), dim3(grid), dim3(kThreads), 0, s, b, bytes, sink); break;
    case 16: hipLaunchKernelGGL((stream_read_kernel<POL, 16>), dim3(grid), dim3(kThreads), 0, s, b, bytes, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

extern "C" {

/*
 * pa_bench_stream_read - read `bytes` of device memory at `buf` once.
 *   bytes      a positive multiple of 16 KiB, below 2^31 (one buffer resource).
 *   policy     0 default cache policy, 1 non-temporal (streaming).
 *   unroll     16-byte loads in flight per lane and round: 4, 8 or 16.
 *   grid       workgroups of 256 threads (4 wavefronts); the caller sizes it from the CU count.
 *   sink       device memory of grid * 4 * 64 * 4 bytes, written (contents meaningless).
 * Returns 0, or a nonzero code for bad arguments (nothing launched) or a launch error.
 */
int pa_bench_stream_read(const void* buf, uint64_t bytes, int policy, int unroll, int grid, void* sink,
                         void* stream) {
  if (!buf || !sink || grid <= 0 || bytes == 0 || bytes % 16384 != 0 || bytes >= (1ull << 31)) return 1;
  if (policy != 0 && policy != 1) return 1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t* out = static_cast<uint32_t*>(sink);
  const hipError_t e = policy == 0 ? launch_pol<0>(unroll, buf, (uint32_t)bytes, grid, out, s)
                                   : launch_pol<2>(unroll, buf, (uint32_t)bytes, grid, out, s);
  return e == hipSuccess ? 0 : 2;
}

}  // extern "C"
