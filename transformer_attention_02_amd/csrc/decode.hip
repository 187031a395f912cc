// KV-cache decode: cache append, split-KV partial attention, log-sum-exp merge.
//
// The new token of sequence b sits at position L = lens[b]. Its key is rotated
// at L and written with its value at cache slot L (a cache pre-allocated and
// written by position, as the roadmap of "Building Grouped-Query Attention with
// RoPE and Flash Attention from Scratch" describes); its query, rotated at L,
// attends slots 0..L. Keys are cut into splits of kDecodeSplit slots; each split
// yields an unnormalised partial output with its running max m and denominator
// l, and the merge combines them with weights 2^(m_s - M): the same rescaling
// rule as the online-softmax recurrences of "Building a Transformer from
// Scratch", Part 3, applied across splits instead of along one loop.
#include "attn_internal.h"

namespace attn {

namespace {

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.4426950408889634f;

template <int BF16>
__device__ __forceinline__ float ld(const void* base, long i) {
  if constexpr (BF16) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
  } else {
    return reinterpret_cast<const float*>(base)[i];
  }
}

__device__ __forceinline__ bool bad_len(int L, int Lmax) { return L < 0 || L >= Lmax; }

// Grid (KV, B), hd/2 threads: rotate k_new at L and write slot L of both caches.
template <int BF16>
__global__ void decode_append_kernel(DecodeArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, p = threadIdx.x;
  const int L = a.lens[b];
  if (bad_len(L, a.Lmax) || 2 * p >= a.hd) return;
  const long src = ((long)b * a.KV + g) * a.hd + 2 * p;
  const long dst = (((long)b * a.KV + g) * a.Lmax + L) * a.hd + 2 * p;
  float x0 = ld<BF16>(a.k_new, src), x1 = ld<BF16>(a.k_new, src + 1);
  if (a.rope) {
    float c, s;
    rope_cos_sin(L, a.freqs.rev[p], c, s);
    const float y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
    x0 = y0;
    x1 = y1;
  }
  if constexpr (BF16) {
    reinterpret_cast<uint32_t*>(a.k_cache)[dst >> 1] = pack_bf16x2(x0, x1);
    reinterpret_cast<uint32_t*>(a.v_cache)[dst >> 1] = reinterpret_cast<const uint32_t*>(a.v_new)[src >> 1];
  } else {
    reinterpret_cast<float2*>(a.k_cache)[dst >> 1] = make_float2(x0, x1);
    reinterpret_cast<float2*>(a.v_cache)[dst >> 1] = reinterpret_cast<const float2*>(a.v_new)[src >> 1];
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Vector-ALU split kernel. Grid (nsplit, H, B), 256 threads: thread = key slot
// for the scores, thread = head-dim index for the partial output.
template <int BF16, int HD>
__global__ __launch_bounds__(256) void decode_split_valu_kernel(DecodeArgs a) {
  constexpr int C = kDecodeSplit;
  static_assert(C == 256, "one key per thread");
  const int sp = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = a.lens[b];
  if (bad_len(L, a.Lmax)) return;
  const int k0 = sp * C;
  if (k0 > L) return;
  const int k1 = min(L + 1, k0 + C);
  const int g = h / a.group;
  const int t = threadIdx.x;
  __shared__ float qs[HD];
  __shared__ float ps[C];
  __shared__ float red[4];

  if (t < HD / 2) {
    const long qi = ((long)b * a.H + h) * HD + 2 * t;
    float x0 = ld<BF16>(a.q, qi), x1 = ld<BF16>(a.q, qi + 1);
    if (a.rope) {
      float c, s;
      rope_cos_sin(L, a.freqs.rev[t], c, s);
      const float y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
      x0 = y0;
      x1 = y1;
    }
    qs[2 * t] = x0 * a.scale_log2;
    qs[2 * t + 1] = x1 * a.scale_log2;
  }
  __syncthreads();
  const long cbase = ((long)b * a.KV + g) * (long)a.Lmax * HD;
  const float slope2 = a.alibi ? alibi_slope(a.alibi, h, a.H) * kLog2e : 0.f;
  const int key = k0 + t;
  float x = -INFINITY;
  if (key < k1) {
    float dot = 0.f;
    for (int d = 0; d < HD; ++d) dot = fmaf(qs[d], ld<BF16>(a.k_cache, cbase + (long)key * HD + d), dot);
    x = dot - slope2 * (float)(L - key);
  }
  const int w = t >> 6, lane = t & 63;
  float mx = wave_max(x);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float p = (key < k1) ? exp2f(x - mx) : 0.f;
  ps[t] = p;
  __syncthreads();
  float sm = wave_sum(p);
  __syncthreads();
  if (lane == 0) red[w] = sm;
  __syncthreads();
  sm = red[0] + red[1] + red[2] + red[3];
  const long pidx = ((long)b * a.H + h) * a.nsplit + sp;
  if (t < HD) {
    float o = 0.f;
    for (int j = 0; j < k1 - k0; ++j) o = fmaf(ps[j], ld<BF16>(a.v_cache, cbase + (long)(k0 + j) * HD + t), o);
    a.part_o[pidx * HD + t] = o;
  }
  if (t == 0) a.part_ml[pidx] = make_float2(mx, sm);
}

// Merge the partials of one (b, h). Grid (H, B), hd threads.
template <int HD>
__global__ void decode_merge_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int L = a.lens[b];
  const long orow = ((long)b * a.H + h) * HD;
  float res, lse;
  if (bad_len(L, a.Lmax)) {
    res = __builtin_nanf("");
    lse = res;
  } else {
    const int ns = (L + 1 + kDecodeSplit - 1) / kDecodeSplit;
    const long p0 = ((long)b * a.H + h) * a.nsplit;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, a.part_ml[p0 + s].x);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float2 ml = a.part_ml[p0 + s];
      const float wgt = exp2f(ml.x - M);
      num = fmaf(wgt, a.part_o[(p0 + s) * HD + d], num);
      den = fmaf(wgt, ml.y, den);
    }
    res = num / den;
    lse = (M + log2f(den)) * kLn2;
  }
  if (a.out_bf16) {
    reinterpret_cast<uint16_t*>(a.out)[orow + d] = f32_to_bf16_bits(res);
  } else {
    reinterpret_cast<float*>(a.out)[orow + d] = res;
  }
  if (a.lse && d == 0) a.lse[(long)b * a.H + h] = lse;
}

template <int BF16, int HD>
hipError_t launch_decode_hd(const DecodeArgs& a, hipStream_t s, const TimingHook& tm) {
  hipLaunchKernelGGL(decode_append_kernel<BF16>, dim3(a.KV, a.B), dim3(HD / 2), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = tm.before(s)) != hipSuccess) return e;
  hipLaunchKernelGGL((decode_split_valu_kernel<BF16, HD>), dim3(a.nsplit, a.H, a.B), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = tm.after(s)) != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<HD>), dim3(a.H, a.B), dim3(HD), 0, s, a);
  return hipGetLastError();
}

template <int BF16>
hipError_t launch_decode_dt(const DecodeArgs& a, hipStream_t s, const TimingHook& tm) {
  switch (a.hd) {
    case 8: return launch_decode_hd<BF16, 8>(a, s, tm);
    case 16: return launch_decode_hd<BF16, 16>(a, s, tm);
    case 32: return launch_decode_hd<BF16, 32>(a, s, tm);
    case 64: return launch_decode_hd<BF16, 64>(a, s, tm);
    case 128: return launch_decode_hd<BF16, 128>(a, s, tm);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int bf16, hipStream_t s, const TimingHook& tm) {
  return bf16 ? launch_decode_dt<1>(a, s, tm) : launch_decode_dt<0>(a, s, tm);
}

}  // namespace attn
