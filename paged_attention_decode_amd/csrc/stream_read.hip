// Practical ceilings for the benchmark (measurement only; built as its own library,
// libpa_stream_read.so, and not part of libpagedattn's ABI): a streaming read for the decode
// kernel's HBM bound and a matrix-core loop for the prefill kernel's MFMA bound.
//
// Streaming read. Reads a large device buffer once with the loads the decode kernel uses for K/V
// pages: 16-byte buffer loads, every lane of a wavefront on consecutive 16-byte chunks (1 KiB per
// load instruction), with the default or the non-temporal cache policy. Each wavefront keeps
// UNROLL such loads in flight per round and walks the buffer with a stride of all wavefronts'
// rounds. The loaded words are summed into one 32-bit word per lane and written to `sink`, so no
// load is dead; the sink is 256 bytes per wavefront, negligible next to the buffer.
//
// The rate this kernel reaches is the practical HBM read ceiling of the GPU for this access
// pattern: the decode kernel's K/V bandwidth is reported as a fraction of it as well as of the
// 8 TB/s peak.
//
// Matrix-core loop. Every wavefront issues `iters` rounds of eight independent matrix-core
// instructions of one kind (the prefill kernel's 16x16x32 bf16 / fp16 forms, or the decode
// kernel's 16x16x16 bf16 form) on register operands, eight accumulator chains so that no
// instruction waits for the previous one's result. Nothing else runs, so the rate it reaches, at
// whatever clock the GPU holds under that load, is the practical matrix-core ceiling. The caller
// may ask for unused LDS per workgroup, which caps how many workgroups share a compute unit and so
// spreads the grid evenly over the compute units.

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

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 h8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef short s4 __attribute__((__vector_size__(4 * sizeof(short))));

template <int KIND>
__device__ __forceinline__ f4 mfma(u4 a, u4 b, f4 c) {
  if constexpr (KIND == 0) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
  } else if constexpr (KIND == 1) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
  } else {
    const s4 a2 = __builtin_bit_cast(s4, __builtin_shufflevector(a, a, 0, 1));
    const s4 b2 = __builtin_bit_cast(s4, __builtin_shufflevector(b, b, 0, 1));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a2, b2, c, 0, 0, 0);
  }
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(int iters, uint32_t seed, float* sink) {
  const int lane = threadIdx.x & 63;
  const uint32_t wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  // Small finite operands that depend on the lane and on a kernel argument, so nothing folds.
  const uint32_t w = ((seed + (uint32_t)lane) & 0x7Fu) | 0x3C00u;  // fp16 / bf16 bits in [1, 2)
  const u4 a = u4{w | (w << 16), w | (w << 16), w | (w << 16), w | (w << 16)};
  const u4 b = u4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u} ^ u4{seed & 1u, 0u, 0u, 0u};
  f4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = mfma<KIND>(a, b, acc[i]);
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) sum += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  sink[(uint64_t)wave * 64 + lane] = sum;
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

/*
 * pa_bench_mfma - matrix-core loop: every wavefront of `grid` workgroups (256 threads, 4
 * wavefronts) issues iters * 8 instructions of one kind:
 *   kind 0  v_mfma_f32_16x16x32_bf16   (16384 flops each)
 *   kind 1  v_mfma_f32_16x16x32_f16    (16384 flops each)
 *   kind 2  v_mfma_f32_16x16x16_bf16   (8192 flops each)
 *   lds_bytes  unused LDS requested per workgroup (at most 65536), to cap the workgroups a
 *           compute unit holds: 65536 allows two of them on gfx950's 160 KiB.
 *   sink    device memory of grid * 256 * 4 bytes, written (contents meaningless).
 * Returns 0, or a nonzero code for bad arguments (nothing launched) or a launch error.
 */
int pa_bench_mfma(int kind, int iters, int grid, int lds_bytes, void* sink, void* stream) {
  if (!sink || grid <= 0 || iters <= 0 || kind < 0 || kind > 2 || lds_bytes < 0 || lds_bytes > 65536) return 1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* out = static_cast<float*>(sink);
  const uint32_t seed = 0x35u;
  const size_t lds = (size_t)lds_bytes;
  if (kind == 0) hipLaunchKernelGGL((mfma_loop_kernel<0>), dim3(grid), dim3(kThreads), lds, s, iters, seed, out);
  if (kind == 1) hipLaunchKernelGGL((mfma_loop_kernel<1>), dim3(grid), dim3(kThreads), lds, s, iters, seed, out);
  if (kind == 2) hipLaunchKernelGGL((mfma_loop_kernel<2>), dim3(grid), dim3(kThreads), lds, s, iters, seed, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
