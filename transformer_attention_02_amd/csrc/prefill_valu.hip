// Rotary pre-pass for keys and the vector-ALU prefill kernel.
//
// The vector-ALU kernel is the path for fp32 inputs (e.g. the 6-token lab
// instance) and for shapes the MFMA kernel does not take. It runs the same
// tiled online softmax as the MFMA kernel ("Building Grouped-Query Attention
// with RoPE and Flash Attention from Scratch", Step 3; the running max /
// denominator recurrences of "Building a Transformer from Scratch", Part 3),
// with all arithmetic in fp32.
#include "attn_internal.h"

namespace attn {

namespace {

template <int BF16>
__device__ __forceinline__ float ld(const void* base, long i) {
  if constexpr (BF16) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
  } else {
    return reinterpret_cast<const float*>(base)[i];
  }
}

// Rotate every key row once: row (b, g) token t sits at position pos0 + t.
// A thread owns one (token, 16-byte chunk) and rotates that chunk in kRopeRows
// consecutive (b, g) rows, so the cos/sin of its pairs are computed once and
// reused; all loads are issued before the stores. Output keeps the input type
// (bf16 rounded to nearest even, exactly as a rotated tile would be rounded
// before an MFMA contraction).
constexpr int kRopeRows = 8;

template <int BF16>
__global__ __launch_bounds__(256) void rope_k_kernel(RopeKArgs a) {
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int chunks = a.hd / EPC;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)a.T * chunks) return;
  const int t = (int)(idx / chunks), c = (int)(idx % chunks);
  float cs[EPC / 2], sn[EPC / 2];
#pragma unroll
  for (int p = 0; p < EPC / 2; ++p) rope_cos_sin(a.pos0 + t, a.freqs.rev[c * (EPC / 2) + p], cs[p], sn[p]);
  const int r0 = blockIdx.y * kRopeRows;
  const uint4* __restrict__ src = reinterpret_cast<const uint4*>(a.k);
  uint4* __restrict__ dst = reinterpret_cast<uint4*>(a.kr);
  uint4 x[kRopeRows];
#pragma unroll
  for (int j = 0; j < kRopeRows; ++j) {
    const long e = (((long)(r0 + j) * a.T + t) * a.hd + (long)c * EPC) / EPC;
    x[j] = (r0 + j < a.heads) ? src[e] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kRopeRows; ++j) {
    if (r0 + j >= a.heads) break;
    const long e = (((long)(r0 + j) * a.T + t) * a.hd + (long)c * EPC) / EPC;
    uint4 y;
    if constexpr (BF16) {
      uint32_t w[4] = {x[j].x, x[j].y, x[j].z, x[j].w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x0 = bf16_bits_to_f32(w[p] & 0xffffu), x1 = bf16_bits_to_f32(w[p] >> 16);
        w[p] = pack_bf16x2(rot0(x0, x1, cs[p], sn[p]), rot1(x0, x1, cs[p], sn[p]));
      }
      y = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      const float f0 = __uint_as_float(x[j].x), f1 = __uint_as_float(x[j].y);
      const float f2 = __uint_as_float(x[j].z), f3 = __uint_as_float(x[j].w);
      y = make_uint4(__float_as_uint(rot0(f0, f1, cs[0], sn[0])), __float_as_uint(rot1(f0, f1, cs[0], sn[0])),
                     __float_as_uint(rot0(f2, f3, cs[1], sn[1])), __float_as_uint(rot1(f2, f3, cs[1], sn[1])));
    }
    dst[e] = y;
  }
}

// One workgroup of 64 threads per (64-query block, head, batch); thread = query row.
// K/V tiles of 64 keys are staged in LDS as fp32 and read by broadcast; the
// online softmax runs in log2 units (q carries log2(e)/sqrt(hd)).
template <int BF16, int HD>
__global__ __launch_bounds__(64) void prefill_valu_kernel(PrefillArgs a) {
  constexpr int BQ = 64, BK = 64, SUB = 16;
  __shared__ float ks[BK][HD];
  __shared__ float vs[BK][HD];
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / a.group;
  const int t = threadIdx.x;
  const int i = qb * BQ + t;
  const bool active = i < a.Tq;
  const int ti = a.q_off + i;  // this query's token index in the key sequence
  const long qrow = (((long)b * a.H + h) * a.Tq + (active ? i : 0)) * HD;
  const long kvbase = ((long)b * a.KV + g) * (long)a.Tk * HD;

  float q[HD], acc[HD];
#pragma unroll
  for (int p = 0; p < HD / 2; ++p) {
    const float x0 = ld<BF16>(a.q, qrow + 2 * p), x1 = ld<BF16>(a.q, qrow + 2 * p + 1);
    float y0 = x0, y1 = x1;
    if (a.rope) {
      float c, s;
      rope_cos_sin(a.pos0 + ti, a.freqs.rev[p], c, s);
      y0 = rot0(x0, x1, c, s);
      y1 = rot1(x0, x1, c, s);
    }
    q[2 * p] = y0 * a.scale_log2;
    q[2 * p + 1] = y1 * a.scale_log2;
    acc[2 * p] = 0.f;
    acc[2 * p + 1] = 0.f;
  }
  const float slope2 = a.alibi ? alibi_slope(a.alibi, h, a.H) * 1.4426950408889634f : 0.f;
  float m = -INFINITY, l = 0.f;

  // key tiles the block's rows can see: up to the last row's token (causal),
  // from the first row's window start (sliding window)
  const int ntiles_all = (a.Tk + BK - 1) / BK;
  const int t_last = a.q_off + min(a.Tq, qb * BQ + BQ) - 1;
  const int ntiles = a.causal ? min(t_last / BK + 1, ntiles_all) : ntiles_all;
  const int kt0 = a.window ? max(0, a.q_off + qb * BQ - a.window + 1) / BK : 0;
  for (int kt = kt0; kt < ntiles; ++kt) {
    __syncthreads();
    for (int e = t; e < BK * HD; e += 64) {
      const int r = e / HD, d = e - r * HD;
      const int key = kt * BK + r;
      const bool in = key < a.Tk;
      ks[r][d] = in ? ld<BF16>(a.k, kvbase + (long)key * HD + d) : 0.f;
      vs[r][d] = in ? ld<BF16>(a.v, kvbase + (long)key * HD + d) : 0.f;
    }
    __syncthreads();
    if (!active) continue;
    for (int j0 = 0; j0 < BK; j0 += SUB) {
      float sc[SUB];
      float mt = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < SUB; ++jj) {
        const int key = kt * BK + j0 + jj;
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < HD; ++d) dot = fmaf(q[d], ks[j0 + jj][d], dot);
        const int dist = ti - key;
        const bool vis = key < a.Tk && (!a.causal || dist >= 0) && (!a.window || dist < a.window);
        const float x = dot - slope2 * (float)(dist < 0 ? -dist : dist);
        sc[jj] = vis ? x : -INFINITY;
        mt = fmaxf(mt, sc[jj]);
      }
      const float m_new = fmaxf(m, mt);
      if (m_new == -INFINITY) continue;  // nothing visible yet in this row
      const float alpha = exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < HD; ++d) acc[d] *= alpha;
#pragma unroll
      for (int jj = 0; jj < SUB; ++jj) {
        const float p = exp2f(sc[jj] - m_new);
        l += p;
#pragma unroll
        for (int d = 0; d < HD; ++d) acc[d] = fmaf(p, vs[j0 + jj][d], acc[d]);
      }
      m = m_new;
    }
  }
  if (!active) return;
  const float inv_l = 1.0f / l;
  const long orow = (((long)b * a.H + h) * a.Tq + i) * HD;
  if (a.out_bf16) {
    uint32_t* o = reinterpret_cast<uint32_t*>(a.out) + (orow >> 1);
#pragma unroll
    for (int p = 0; p < HD / 2; ++p) o[p] = pack_bf16x2(acc[2 * p] * inv_l, acc[2 * p + 1] * inv_l);
  } else {
    float* o = reinterpret_cast<float*>(a.out) + orow;
#pragma unroll
    for (int d = 0; d < HD; ++d) o[d] = acc[d] * inv_l;
  }
  if (a.lse) a.lse[((long)b * a.H + h) * a.Tq + i] = (m + log2f(l)) * 0.69314718055994531f;
}

template <int BF16>
hipError_t launch_valu_hd(const PrefillArgs& a, hipStream_t s) {
  dim3 grid((a.Tq + 63) / 64, a.H, a.B);
  switch (a.hd) {
    case 8: hipLaunchKernelGGL((prefill_valu_kernel<BF16, 8>), grid, dim3(64), 0, s, a); break;
    case 16: hipLaunchKernelGGL((prefill_valu_kernel<BF16, 16>), grid, dim3(64), 0, s, a); break;
    case 32: hipLaunchKernelGGL((prefill_valu_kernel<BF16, 32>), grid, dim3(64), 0, s, a); break;
    case 64: hipLaunchKernelGGL((prefill_valu_kernel<BF16, 64>), grid, dim3(64), 0, s, a); break;
    case 128: hipLaunchKernelGGL((prefill_valu_kernel<BF16, 128>), grid, dim3(64), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_k(const RopeKArgs& a, int bf16, hipStream_t s) {
  const long items = (long)a.T * (a.hd / (bf16 ? 8 : 4));
  dim3 grid((unsigned)((items + 255) / 256), (unsigned)((a.heads + kRopeRows - 1) / kRopeRows));
  if (bf16) {
    hipLaunchKernelGGL(rope_k_kernel<1>, grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(rope_k_kernel<0>, grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_valu(const PrefillArgs& a, int bf16, hipStream_t s) {
  return bf16 ? launch_valu_hd<1>(a, s) : launch_valu_hd<0>(a, s);
}

}  // namespace attn
