// Peak probes for gfx950, used by the benchmark to report the attention
// kernels' rates against what this GPU measurably reaches, next to the
// published MI355X peaks.  Not part of the attention library: built into
// liblazyattn_probe.so.
//
//  - lazyattn_probe_mfma_bf16: every wave runs `iters` rounds of eight
//    independent v_mfma_f32_32x32x16_bf16 accumulation chains (no chain waits
//    on another), so the matrix pipes stay busy; 2 * 32 * 32 * 16 flops each.
//  - lazyattn_probe_hbm_read: a grid-stride streaming read of n 16-byte words,
//    folded into one value per thread (so no load is dropped).
//  - lazyattn_probe_gather_read: work-groups read whole chunks (chunk_bytes, a
//    multiple of 4 KiB) at caller-given offsets, four in flight each: the access
//    pattern of a paged KV pool whose blocks sit at scattered positions.
//
// Each thread stores its result to its own slot of `sink` (vector stores).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(0.001f * static_cast<float>((lane + i) & 7));
    b[i] = static_cast<__bf16>(0.002f * static_cast<float>((lane * 3 + i) & 7));
  }
  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void hbm_read_kernel(const uint4* src, size_t n, float* sink) {
  const size_t tid = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  uint32_t x = 0;
  size_t i = tid;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    x ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
    x ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  for (; i < n; i += stride) {
    const uint4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[tid] = static_cast<float>(x & 0xffu);
}

// Work-group b reads chunks 4b .. 4b + 3, then 4(b + gridDim.x) .., of the offset
// list, four chunks in flight at a time; each chunk is read 4 KiB at a time, 16
// bytes per thread.
__global__ __launch_bounds__(256) void gather_read_kernel(const uint4* base, const int64_t* offsets, int n_chunks,
                                                          int chunk_units, float* sink) {
  uint32_t x = 0;
  for (int c = 4 * blockIdx.x; c < n_chunks; c += 4 * gridDim.x) {
    const uint4* p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = base + offsets[min(c + j, n_chunks - 1)] / 16;
    for (int u = 0; u < chunk_units; ++u) {
      uint4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = p[j][u * 256 + threadIdx.x];
#pragma unroll
      for (int j = 0; j < 4; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
  }
  sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = static_cast<float>(x & 0xffu);
}

}  // namespace

extern "C" {

// FLOPs issued by one call: num_wg * 4 waves * iters * 8 chains * 32768.
// sink: device float [num_wg * 256].  0 on success, else the HIP error code.
int lazyattn_probe_mfma_bf16(int num_wg, int iters, float* sink, hipStream_t stream) {
  if (num_wg < 1 || iters < 1 || !sink) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(num_wg), dim3(256), 0, stream, iters, sink);
  return static_cast<int>(hipGetLastError());
}

// Reads n 16-byte words of src (device).  sink: device float [num_wg * 256].
int lazyattn_probe_hbm_read(const void* src, size_t n, int num_wg, float* sink, hipStream_t stream) {
  if (num_wg < 1 || !src || !sink) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(hbm_read_kernel, dim3(num_wg), dim3(256), 0, stream, static_cast<const uint4*>(src), n, sink);
  return static_cast<int>(hipGetLastError());
}

// Reads n_chunks chunks of chunk_bytes (a multiple of 4096) at byte offsets
// offsets[i] (device int64, multiples of 16) from base (device).  sink: device
// float [num_wg * 256].
int lazyattn_probe_gather_read(const void* base, const int64_t* offsets, int n_chunks, int chunk_bytes, int num_wg,
                               float* sink, hipStream_t stream) {
  if (num_wg < 1 || n_chunks < 0 || chunk_bytes < 4096 || chunk_bytes % 4096 != 0 || !base || !offsets || !sink)
    return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(gather_read_kernel, dim3(num_wg), dim3(256), 0, stream, static_cast<const uint4*>(base), offsets,
                     n_chunks, chunk_bytes / 4096, sink);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
