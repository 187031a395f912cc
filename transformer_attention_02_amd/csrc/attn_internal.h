// Internal declarations shared by the HIP translation units of libattn.so.
// Nothing here is part of the C ABI (include/attn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

constexpr int kMaxHeadDim = 128;
constexpr int kDecodeSplit = 256;  // keys per split-KV partial, vector-ALU decode kernel
constexpr int kSplitMfma = 512;    // keys per split-KV partial, MFMA decode kernel
constexpr int kSplitMfmaLong = 1024;  // the same when the batch gives enough splits anyway
constexpr int kSplitMfmaFp8 = 2048;   // fp8 cache: the same bytes per workgroup as the long bf16 split
constexpr int kMaxDecodeLmax = 1 << 24;  // cache slots per sequence the decode entry points accept

// 4 theta_i / (2 pi) in fp64 (quarter turns per position) for i = 0 .. hd/2-1,
// theta_i = base^(-2i/hd).
// Passed by value so the kernels need no table in device memory.
struct RopeFreqs {
  double rev[kMaxHeadDim / 2];
};

struct PrefillArgs {
  const void* q;     // [B,H,Tq,hd]
  const void* k;     // [B,KV,Tk,hd] rotated keys (workspace) or raw keys when rope is off
  const void* v;     // [B,KV,Tk,hd]
  void* out;         // [B,H,Tq,hd]
  float* lse;        // [B,H,Tq] or nullptr
  int B, Tq, Tk, H, KV, hd, group;
  int pos0;          // position of key token 0
  int q_off;         // query row i is key token q_off + i (q_off + Tq <= Tk)
  int window;        // > 0: a query sees only its last `window` tokens (causal only)
  int causal;
  int rope;
  int alibi;
  int out_bf16;
  float scale_log2;  // log2(e) / sqrt(hd)
  RopeFreqs freqs;
};

struct RopeKArgs {
  const void* k;  // [heads, T, hd] raw
  void* kr;       // [heads, T, hd] rotated
  int heads;      // B*KV
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
  int B, H, KV, hd, group, Lmax;
  int split;             // key slots per partial
  int nsplit;            // partial slots per (b, h): ceil(Lmax / split)
  int rope;
  int alibi;
  int out_bf16;
  float scale_log2;
  RopeFreqs freqs;
  int fp8;               // caches hold OCP E4M3 codes (value = code * scale)
  float k_scale, v_scale;
  int append;            // 1: write k_new/v_new to slot L; 0: slot L already holds them
};

// Latent-attention decode (cache of one d_c-dim latent per token, shared by all heads).
constexpr int kLatentSplit = 512;        // keys per split-KV partial (whole 16-key tiles)
constexpr int kLatentMaxSplits = 512;    // splits per sequence the merge handles
struct LatentArgs {
  const void* q;         // [B,H,hd] bf16
  const void* c_new;     // [B,dc] bf16
  void* c_cache;         // [B,Lmax,dc] bf16
  const int32_t* lens;   // [B]
  const void* w_uk;      // [H,dc,hd] bf16
  const void* w_uv;      // [H,dc,hd] bf16
  void* out;             // [B,H,hd]
  float* lse;            // [B,H] or nullptr
  uint16_t* qt;          // [B,H,dc] bf16 folded queries (workspace)
  float* part_o;         // [B,H,nsplit,dc] (workspace)
  float2* part_ml;       // [B,H,nsplit]
  float* ot;             // [B,H,dc] merged latent outputs (workspace)
  int* items;            // [B*nsplit + 1] (workspace): active (sequence, split) pairs, then their count
  int B, H, hd, dc, Lmax;
  int hblocks;           // ceil(H / 16)
  int split, nsplit;
  int alibi, out_bf16;
  float scale_log2;      // log2(e) / sqrt(hd)
};

struct BwdArgs {
  const void* q;     // [B,H,T,hd] rotated queries (workspace) or raw when rope is off
  const void* k;     // [B,KV,T,hd] rotated keys (workspace) or raw
  const void* v;     // [B,KV,T,hd]
  const void* dout;  // [B,H,T,hd] (out dtype)
  const float* lse;  // [B,H,T] natural-log log-sum-exp from the forward
  const void* out;   // [B,H,T,hd] forward output (out_dtype)
  float* D;          // [B,H,T] rowsum(dout * out) (workspace)
  void* dq;          // [B,H,T,hd] (grad dtype)
  void* dk;          // [B,KV,T,hd]
  void* dv;          // [B,KV,T,hd]
  int B, T, H, KV, hd, group;
  int pos0;
  int causal;
  int rope;
  int alibi;
  int in_bf16;       // q, k, v
  int out_bf16;      // out, dout
  int grad_bf16;     // dq, dk, dv
  float scale;       // 1 / sqrt(hd)
  RopeFreqs freqs;
};

struct BwdPrepArgs {
  const void* out;   // [rows, hd]
  const void* dout;  // [rows, hd]
  float* D;          // [rows]
  long rows;
  int hd;
  int out_bf16;
};

// Events recorded around the main kernel of one call (either may be null).
struct TimingHook {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
  hipError_t before(hipStream_t s) const { return start ? hipEventRecord(start, s) : hipSuccess; }
  hipError_t after(hipStream_t s) const { return stop ? hipEventRecord(stop, s) : hipSuccess; }
};

hipError_t launch_rope_k(const RopeKArgs& a, int bf16, hipStream_t s);
hipError_t launch_prefill_valu(const PrefillArgs& a, int bf16, hipStream_t s);
bool prefill_mfma_supported(const PrefillArgs& a, int bf16);
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int bf16, hipStream_t s, const TimingHook& tm);
bool decode_mfma_supported(const DecodeArgs& a, int bf16);
int decode_split_for(const DecodeArgs& a, int bf16);  // key slots per split the launcher uses
hipError_t launch_bwd_prep(const BwdPrepArgs& a, hipStream_t s);
hipError_t launch_bwd_valu(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dkv_valu(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dq_mfma(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dkv_mfma(const BwdArgs& a, hipStream_t s);
bool bwd_mfma_supported(const BwdArgs& a);
hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t s, const TimingHook& tm);
hipError_t launch_decode_latent(const LatentArgs& a, hipStream_t s, const TimingHook& tm);

// ---------------------------------------------------------------- device helpers
#if defined(__HIPCC__)
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));  // round to nearest even
}

// Two floats -> two bf16 packed in one dword (low half = lo), round to nearest
// even, with one v_cvt_pk_bf16_f32.
typedef float attn_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 attn_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const attn_f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, attn_bf16x2));
}

// Raw buffer descriptor over [base, base + bytes) (gfx9-family word 3). Buffer
// loads through it return zero for any lane whose offset is at or past `bytes`,
// so a descriptor that starts at a tile and ends at the end of the tensor slab
// zero-fills rows past the sequence end without per-lane address checks.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voffset) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 0));
}
// The same load marked non-temporal (gfx950 cache-policy bit "nt", aux = 2):
// for data read exactly once, such as a KV cache streamed by decode (measured:
// about 12% more read bandwidth than the default policy).
__device__ __forceinline__ uint4 buffer_load16_stream(__amdgpu_buffer_rsrc_t r, int voffset) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 2));
}

// cos/sin of the rotary angle pos * theta, with q4 = 4 * theta / (2 pi) in fp64
// (the angle in quarter turns per position). The angle is reduced in fp64 to a
// quadrant k and a remainder f in [-pi/4, pi/4]; sin f and cos f are the Taylor
// series to degree 9 and 8 (truncation below 3e-8 on that interval), and the
// quadrant rotates the pair. Accurate to fp32 rounding for any position.
__device__ __forceinline__ void rope_cos_sin(int pos, double q4, float& c, float& s) {
  const double x = (double)pos * q4;
  const double k = rint(x);
  const float f = (float)((x - k) * 1.5707963267948966);
  const float f2 = f * f;
  const float sf = f * fmaf(f2, fmaf(f2, fmaf(f2, fmaf(f2, 2.7557319223985893e-6f, -1.9841269841269841e-4f),
                                                 8.3333333333333333e-3f), -1.6666666666666667e-1f), 1.0f);
  const float cf = fmaf(f2, fmaf(f2, fmaf(f2, fmaf(f2, 2.4801587301587302e-5f, -1.3888888888888889e-3f),
                                          4.1666666666666667e-2f), -0.5f), 1.0f);
  const int q = (int)((long long)k & 3);
  const float s1 = (q & 1) ? cf : sf;
  const float c1 = (q & 1) ? sf : cf;
  s = (q & 2) ? -s1 : s1;
  c = ((q + 1) & 2) ? -c1 : c1;
}

// Rotate the pair (x0, x1) by the angle with cosine c and sine s. Written with
// explicit FMAs so every kernel rounds the rotation identically (the compiler
// may not contract these differently in different call sites).
__device__ __forceinline__ float rot0(float x0, float x1, float c, float s) { return fmaf(x0, c, -(x1 * s)); }
__device__ __forceinline__ float rot1(float x0, float x1, float c, float s) { return fmaf(x0, s, x1 * c); }

// ALiBi slope of head h out of H for the two slope families, in fp32.
__device__ __forceinline__ float alibi_slope(int kind, int h, int H) {
  const float e = (kind == 1 ? -8.0f : -2.0f) * (float)(h + 1) / (float)H;
  return exp2f(e);
}
#endif

}  // namespace attn
