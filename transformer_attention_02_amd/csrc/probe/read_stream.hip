// Read-only HBM stream for the benchmark's same-run bandwidth ceiling. Not part
// of the attention library: it is built into its own libattn_probe.so.
//
// Every byte of [p, p + bytes) is read once with non-temporal 16-byte loads
// (the cache policy the decode kernels use for their KV streams), eight loads
// in flight per thread; each thread folds what it read into one word and each
// workgroup writes one word to sink, so nothing but the reads reaches memory.
// The launch shape is the fastest of a sweep on MI355X (grid 2048..16384 x 256
// or 512 threads x 4, 8 or 16 loads in flight, with and without the
// non-temporal policy): 16384 x 512 x 8 read 7.1 TB/s, where 2048 x 256 x 4 read
// 6.0 TB/s and plain loads at most 6.1 TB/s.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 512;
constexpr int kGrid = 16384;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4* __restrict__ p, size_t n16,
                                                               unsigned* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  unsigned acc = 0;
  constexpr int NL = 8;
  for (; i + (NL - 1) * stride < n16; i += NL * stride) {
    u32x4 v[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) v[j] = __builtin_nontemporal_load(p + i + j * stride);
#pragma unroll
    for (int j = 0; j < NL; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ unsigned red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from device pointer p on `stream`; sink is a
// device buffer of at least attn_probe_sink_words() unsigned words. Returns 0,
// 1 for bad arguments, 2 if the launch fails.
size_t attn_probe_sink_words(void) { return kGrid; }

int attn_probe_read_stream(const void* p, size_t bytes, unsigned* sink, void* stream) {
  if (!p || !sink || bytes % 16 || (reinterpret_cast<uintptr_t>(p) % 16)) return 1;
  hipLaunchKernelGGL(read_stream_kernel, dim3(kGrid), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const u32x4*>(p), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
