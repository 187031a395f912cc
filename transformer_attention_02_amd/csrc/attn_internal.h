// Internal declarations shared by the HIP translation units of libattn.so.
// Nothing here is part of the C ABI (include/attn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

constexpr int kMaxHeadDim = 128;
constexpr int kDecodeSplit = 256;  // keys per split-KV partial in decode

// theta_i / (2 pi) in fp64 for i = 0 .. hd/2-1, theta_i = base^(-2i/hd).
// Passed by value so the kernels need no table in device memory.
struct RopeFreqs {
  double rev[kMaxHeadDim / 2];
};

struct PrefillArgs {
  const void* q;     // [B,H,T,hd]
  const void* k;     // [B,KV,T,hd] rotated keys (workspace) or raw keys when rope is off
  const void* v;     // [B,KV,T,hd]
  void* out;         // [B,H,T,hd]
  float* lse;        // [B,H,T] or nullptr
  int B, T, H, KV, hd, group;
  int pos0;
  int causal;
  int rope;
  int alibi;
  int out_bf16;
  float scale_log2;  // log2(e) / sqrt(hd)
  RopeFreqs freqs;
};

struct RopeKArgs {
  const void* k;  // [rows, hd] raw
  void* kr;       // [rows, hd] rotated
  long rows;      // B*KV*T
  int T, hd, pos0;
  RopeFreqs freqs;
};

struct DecodeArgs {
  const void* q;         // [B,H,hd]
  const void* k_new;     // [B,KV,hd]
  const void* v_new;     // [B,KV,hd]
  void* k_cache;         // [B,KV,Lmax,hd]
  void* v_cache;         // [B,KV,Lmax,hd]
  const int32_t* lens;   // [B]
  void* out;             // [B,H,hd]
  float* lse;            // [B,H] or nullptr
  float* part_o;         // [B,H,nsplit,hd]
  float2* part_ml;       // [B,H,nsplit]  (running max in log2 units, denominator)
  int B, H, KV, hd, group, Lmax, nsplit;
  int rope;
  int alibi;
  int out_bf16;
  float scale_log2;
  RopeFreqs freqs;
};

hipError_t launch_rope_k(const RopeKArgs& a, int bf16, hipStream_t s);
hipError_t launch_prefill_valu(const PrefillArgs& a, int bf16, hipStream_t s);
bool prefill_mfma_supported(const PrefillArgs& a, int bf16);
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int bf16, hipStream_t s);

// ---------------------------------------------------------------- device helpers
#if defined(__HIPCC__)
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));  // round to nearest even
}

// Two floats -> two bf16 packed in one dword (low half = lo), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// cos/sin of the rotary angle pos * theta, where rev = theta / (2 pi) in fp64.
// The angle is reduced to [-pi, pi] in fp64 before the fp32 sincos, so the
// result is accurate to fp32 rounding for any position.
__device__ __forceinline__ void rope_cos_sin(int pos, double rev, float& c, float& s) {
  double a = (double)pos * rev;
  a -= rint(a);
  float r = (float)(a * 6.283185307179586476925286766559);
  sincosf(r, &s, &c);
}

// ALiBi slope of head h out of H for the two slope families, in fp32.
__device__ __forceinline__ float alibi_slope(int kind, int h, int H) {
  const float e = (kind == 1 ? -8.0f : -2.0f) * (float)(h + 1) / (float)H;
  return exp2f(e);
}
#endif

}  // namespace attn
