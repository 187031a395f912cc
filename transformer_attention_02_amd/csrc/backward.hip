// Backward of the prefill forward: rowsum pre-pass and the vector-ALU kernels.
//
// Gradients of sum(out * dout) with respect to q, k and v (the derivative of
// the softmax attention of "Building Grouped-Query Attention with RoPE and
// Flash Attention from Scratch", Step 3; the gradient-flow checks of the
// multi-head and pure-Python pages exercise exactly these). With the rotated
// q', k', the forward's log-sum-exp lse_i and D_i = sum_d dout_id out_id:
//   p_ij  = exp(s_ij - lse_i)                   (recomputed, never stored)
//   dv_j  = sum_i p_ij dout_i
//   ds_ij = p_ij (<dout_i, v_j> - D_i)
//   dq'_i = scale sum_j ds_ij k'_j,  dk'_j = scale sum_i ds_ij q'_i
// and dq = R(-pos) dq', dk = R(-pos) dk' (the rotation is orthogonal).
// D_i equals sum_j p_ij <dout_i, v_j> because out_i = sum_j p_ij v_j.
//
// The vector-ALU kernels (fp32 arithmetic) serve fp32 inputs and head sizes the
// matrix-core kernels do not take: one thread per query row for dq, one per
// key row for dk/dv (looping over the query heads of its group).
#include "attn_internal.h"

namespace attn {

namespace {

constexpr float kLog2eB = 1.4426950408889634f;

template <int BF16>
__device__ __forceinline__ float ldx(const void* base, long i) {
  if constexpr (BF16) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
  } else {
    return reinterpret_cast<const float*>(base)[i];
  }
}

template <int BF16>
__device__ __forceinline__ void stx(void* base, long i, float x) {
  if constexpr (BF16) {
    reinterpret_cast<uint16_t*>(base)[i] = f32_to_bf16_bits(x);
  } else {
    reinterpret_cast<float*>(base)[i] = x;
  }
}

// D_i = sum_d out_id dout_id, one thread per row, 16-byte loads.
template <int OBF16>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdPrepArgs a) {
  const long r = (long)blockIdx.x * 256 + threadIdx.x;
  if (r >= a.rows) return;
  constexpr int EPC = OBF16 ? 8 : 4;  // elements per 16-byte chunk
  const uint4* o = reinterpret_cast<const uint4*>(a.out) + r * a.hd / EPC;
  const uint4* g = reinterpret_cast<const uint4*>(a.dout) + r * a.hd / EPC;
  float acc = 0.f;
  for (int c = 0; c < a.hd / EPC; ++c) {
    const uint4 x = o[c], y = g[c];
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (OBF16) {
        acc = fmaf(bf16_bits_to_f32(xs[w] & 0xffffu), bf16_bits_to_f32(ys[w] & 0xffffu), acc);
        acc = fmaf(bf16_bits_to_f32(xs[w] >> 16), bf16_bits_to_f32(ys[w] >> 16), acc);
      } else {
        acc = fmaf(__uint_as_float(xs[w]), __uint_as_float(ys[w]), acc);
      }
    }
  }
  a.D[r] = acc;
}

// Store a head-dim row of scaled rotated-space gradient g (fp32) back in the
// input frame: pair (2p, 2p+1) rotated by -angle(pos).
template <int GBF16, int HD>
__device__ __forceinline__ void store_unrotated(const BwdArgs& a, void* dst, long row, int pos, const float* g) {
#pragma unroll
  for (int p = 0; p < HD / 2; ++p) {
    const float x0 = g[2 * p] * a.scale, x1 = g[2 * p + 1] * a.scale;
    float y0 = x0, y1 = x1;
    if (a.rope) {
      float c, s;
      rope_cos_sin(pos, a.freqs.rev[p], c, s);
      y0 = rot0(x0, x1, c, -s);
      y1 = rot1(x0, x1, c, -s);
    }
    stx<GBF16>(dst, row + 2 * p, y0);
    stx<GBF16>(dst, row + 2 * p + 1, y1);
  }
}

// dq: one thread per query row; K/V tiles of 32 keys staged in LDS as fp32.
template <int IBF16, int OBF16, int GBF16, int HD>
__global__ __launch_bounds__(64) void bwd_dq_valu_kernel(BwdArgs a) {
  constexpr int BK = 32;
  __shared__ float ks[BK][HD];
  __shared__ float vs[BK][HD];
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int g = h / a.group;
  const int i = qb * 64 + t;
  const bool active = i < a.T;
  const long rowi = ((long)b * a.H + h) * a.T + (active ? i : a.T - 1);
  const long kvbase = ((long)b * a.KV + g) * (long)a.T * HD;
  float qv[HD], dov[HD], dq[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    qv[d] = ldx<IBF16>(a.q, rowi * HD + d);
    dov[d] = ldx<OBF16>(a.dout, rowi * HD + d);
    dq[d] = 0.f;
  }
  const float c2 = a.scale * kLog2eB;
  const float lse2 = a.lse[rowi] * kLog2eB;
  const float Di = a.D[rowi];
  const float slope2 = a.alibi ? alibi_slope(a.alibi, h, a.H) * kLog2eB : 0.f;
  const int kend = a.causal ? min(a.T, qb * 64 + 64) : a.T;
  for (int k0 = 0; k0 < kend; k0 += BK) {
    __syncthreads();
    for (int e = t; e < BK * HD; e += 64) {
      const int r = e / HD, d = e - r * HD;
      const int key = k0 + r;
      const bool in = key < a.T;
      ks[r][d] = in ? ldx<IBF16>(a.k, kvbase + (long)key * HD + d) : 0.f;
      vs[r][d] = in ? ldx<IBF16>(a.v, kvbase + (long)key * HD + d) : 0.f;
    }
    __syncthreads();
    if (!active) continue;
    for (int jj = 0; jj < BK; ++jj) {
      const int key = k0 + jj;
      if (key >= a.T || (a.causal && key > i)) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < HD; ++d) {
        s = fmaf(qv[d], ks[jj][d], s);
        dp = fmaf(dov[d], vs[jj][d], dp);
      }
      const float dist = (float)(i >= key ? i - key : key - i);
      const float p = exp2f(fmaf(s, c2, -slope2 * dist) - lse2);
      const float ds = p * (dp - Di);
#pragma unroll
      for (int d = 0; d < HD; ++d) dq[d] = fmaf(ds, ks[jj][d], dq[d]);
    }
  }
  if (!active) return;
  store_unrotated<GBF16, HD>(a, a.dq, rowi * HD, a.pos0 + i, dq);
}

// dk, dv: one thread per key row, looping over the query heads of its group;
// query tiles of 32 rows (rotated q, dout, lse, D) staged in LDS.
template <int IBF16, int OBF16, int GBF16, int HD>
__global__ __launch_bounds__(64) void bwd_dkv_valu_kernel(BwdArgs a) {
  constexpr int BQ = 32;
  __shared__ float qs[BQ][HD];
  __shared__ float dos[BQ][HD];
  __shared__ float ls[BQ], ds_[BQ];
  const int kb = blockIdx.x, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int j = kb * 64 + t;
  const bool active = j < a.T;
  const long rowj = ((long)b * a.KV + g) * a.T + (active ? j : a.T - 1);
  float kv[HD], vv[HD], dk[HD], dv[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    kv[d] = ldx<IBF16>(a.k, rowj * HD + d);
    vv[d] = ldx<IBF16>(a.v, rowj * HD + d);
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  const float c2 = a.scale * kLog2eB;
  const int qstart = a.causal ? kb * 64 : 0;
  for (int h = g * a.group; h < (g + 1) * a.group; ++h) {
    const float slope2 = a.alibi ? alibi_slope(a.alibi, h, a.H) * kLog2eB : 0.f;
    const long hbase = ((long)b * a.H + h) * a.T;
    for (int q0 = qstart; q0 < a.T; q0 += BQ) {
      __syncthreads();
      for (int e = t; e < BQ * HD; e += 64) {
        const int r = e / HD, d = e - r * HD;
        const int qi = q0 + r;
        const bool in = qi < a.T;
        qs[r][d] = in ? ldx<IBF16>(a.q, (hbase + qi) * HD + d) : 0.f;
        dos[r][d] = in ? ldx<OBF16>(a.dout, (hbase + qi) * HD + d) : 0.f;
      }
      if (t < BQ) {
        const int qi = q0 + t;
        ls[t] = qi < a.T ? a.lse[hbase + qi] * kLog2eB : 0.f;
        ds_[t] = qi < a.T ? a.D[hbase + qi] : 0.f;
      }
      __syncthreads();
      if (!active) continue;
      for (int ii = 0; ii < BQ; ++ii) {
        const int qi = q0 + ii;
        if (qi >= a.T || (a.causal && qi < j)) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < HD; ++d) {
          s = fmaf(qs[ii][d], kv[d], s);
          dp = fmaf(dos[ii][d], vv[d], dp);
        }
        const float dist = (float)(qi >= j ? qi - j : j - qi);
        const float p = exp2f(fmaf(s, c2, -slope2 * dist) - ls[ii]);
        const float dsv = p * (dp - ds_[ii]);
#pragma unroll
        for (int d = 0; d < HD; ++d) {
          dv[d] = fmaf(p, dos[ii][d], dv[d]);
          dk[d] = fmaf(dsv, qs[ii][d], dk[d]);
        }
      }
    }
  }
  if (!active) return;
  store_unrotated<GBF16, HD>(a, a.dk, rowj * HD, a.pos0 + j, dk);
#pragma unroll
  for (int d = 0; d < HD; ++d) stx<GBF16>(a.dv, rowj * HD + d, dv[d]);
}

template <int IBF16, int OBF16, int GBF16, int HD>
hipError_t launch_valu_hd(const BwdArgs& a, hipStream_t s, bool dq, bool dkv) {
  const unsigned nb = (unsigned)((a.T + 63) / 64);
  if (dq) hipLaunchKernelGGL((bwd_dq_valu_kernel<IBF16, OBF16, GBF16, HD>), dim3(nb, a.H, a.B), dim3(64), 0, s, a);
  if (dkv) hipLaunchKernelGGL((bwd_dkv_valu_kernel<IBF16, OBF16, GBF16, HD>), dim3(nb, a.KV, a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int IBF16, int OBF16, int GBF16>
hipError_t launch_valu_g(const BwdArgs& a, hipStream_t s, bool dq, bool dkv) {
  switch (a.hd) {
    case 8: return launch_valu_hd<IBF16, OBF16, GBF16, 8>(a, s, dq, dkv);
    case 16: return launch_valu_hd<IBF16, OBF16, GBF16, 16>(a, s, dq, dkv);
    case 32: return launch_valu_hd<IBF16, OBF16, GBF16, 32>(a, s, dq, dkv);
    case 64: return launch_valu_hd<IBF16, OBF16, GBF16, 64>(a, s, dq, dkv);
    case 128: return launch_valu_hd<IBF16, OBF16, GBF16, 128>(a, s, dq, dkv);
    default: return hipErrorInvalidValue;
  }
}

template <int IBF16, int OBF16>
hipError_t launch_valu_o(const BwdArgs& a, hipStream_t s, bool dq, bool dkv) {
  return a.grad_bf16 ? launch_valu_g<IBF16, OBF16, 1>(a, s, dq, dkv) : launch_valu_g<IBF16, OBF16, 0>(a, s, dq, dkv);
}

template <int IBF16>
hipError_t launch_valu_i(const BwdArgs& a, hipStream_t s, bool dq, bool dkv) {
  return a.out_bf16 ? launch_valu_o<IBF16, 1>(a, s, dq, dkv) : launch_valu_o<IBF16, 0>(a, s, dq, dkv);
}

}  // namespace

hipError_t launch_bwd_prep(const BwdPrepArgs& a, hipStream_t s) {
  const unsigned nb = (unsigned)((a.rows + 255) / 256);
  if (a.out_bf16) {
    hipLaunchKernelGGL(bwd_prep_kernel<1>, dim3(nb), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(bwd_prep_kernel<0>, dim3(nb), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_valu(const BwdArgs& a, hipStream_t s) {
  return a.in_bf16 ? launch_valu_i<1>(a, s, true, true) : launch_valu_i<0>(a, s, true, true);
}

hipError_t launch_bwd_dkv_valu(const BwdArgs& a, hipStream_t s) {
  return a.in_bf16 ? launch_valu_i<1>(a, s, false, true) : launch_valu_i<0>(a, s, false, true);
}

}  // namespace attn
