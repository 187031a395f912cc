// Read-only HBM stream for the benchmark's same-run bandwidth ceiling. Not part
// of the attention library: it is built into its own libattn_probe.so.
//
// Every byte of [p, p + bytes) is read once with non-temporal 16-byte loads
// (the cache policy the decode kernels use for their KV streams), four loads in
// flight per thread; each thread folds what it read into one word and each
// workgroup writes one word to sink, so nothing but the reads reaches memory.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4* __restrict__ p, size_t n16,
                                                               unsigned* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  unsigned acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
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
size_t attn_probe_sink_words(void) { return 2048; }

int attn_probe_read_stream(const void* p, size_t bytes, unsigned* sink, void* stream) {
  if (!p || !sink || bytes % 16 || (reinterpret_cast<uintptr_t>(p) % 16)) return 1;
  hipLaunchKernelGGL(read_stream_kernel, dim3(2048), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const u32x4*>(p), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
