// bf16 matrix-core kernels of the prefill backward (gfx950).
//
// The gradients of sum(out * dout) (see backward.hip for the formulas) are
// split FA2-style into two kernels that never store the attention weights:
//   * dq: a wave owns 32 query rows of one head (the layout of the forward
//     kernel) and streams the K/V tiles: S^T = K Q^T and dP^T = V dO^T on the
//     matrix cores, then P^T = 2^(S^T log2(e)/sqrt(hd) + bias - lse) and
//     dS^T = P^T (dP^T - D) per lane (each lane's query has one lse and one D),
//     and dQ^T += K^T dS^T with dS^T straight from the accumulator registers;
//   * dk/dv: a wave owns 32 keys of one KV head and streams the query rows of
//     every head of the group: S = Q K^T and dP = dO V^T, then
//     dV^T += dO^T P and dK^T += Q^T dS, with P and dS straight from the
//     accumulator registers.
// As in the forward kernel the streamed rows are fed in permuted order (bits 2
// and 3 of the row index swapped) so that accumulator registers 8u..8u+7 hold
// 8 consecutive rows — the B operand of the next contraction — and transposed
// operands come from ds_read_b64_tr_b16. Tiles that are read both as rows and
// transposed are stored with the transposing-read swizzle.
#include <type_traits>

#include "mfma_tile.h"

namespace attn {

namespace {

using namespace tile;

constexpr float kLog2eM = 1.4426950408889634f;

// ------------------------------------------------------------------ dq kernel
constexpr int QW = 4;  // waves per dq workgroup
constexpr int QT = QW * 64;

struct DqGrid {
  int hpw;       // heads per workgroup (1, 2 or 4)
  int hchunks;   // group / hpw
  int bm;        // query rows per head per workgroup = 32 * (QW / hpw)
  int nqb;       // query blocks
  int units;     // B * KV * hchunks
  int xcd_aware;
};

// Per-lane byte offset (from the tile start) of the transposing read for key
// row 8hf + (lane%16)/4 of each 32-column block, for a tile stored with the V
// swizzle. Opaque to the optimiser (see the forward kernel).
template <int HD>
__device__ __forceinline__ void tr_offsets(int lane, int (&off)[HD / 32]) {
  const int li = lane & 15, hf = lane >> 5;
#pragma unroll
  for (int mb = 0; mb < HD / 32; ++mb) {
    const int col = 32 * mb + 16 * ((lane >> 4) & 1) + 4 * (li & 3);
    int o = v_off<HD>(8 * hf + (li >> 2), col >> 3) + (col & 7) * 2;
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(o));
#endif
    off[mb] = o;
  }
}

// A^T operand of 16 rows (16u .. 16u+15 of the tile) x 32 columns (block mb)
// read transposed: lane i of a 16-lane group receives column d0 + i of 4 rows
// per 8-byte load.
template <int HD>
__device__ __forceinline__ bf16x8 read_tr(LdsBytes base, int off, int u) {
  LdsBytes p = base + off + 16 * u * HD * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(p + 4 * HD * 2));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8 pack8(const float* t) {
  return as_bf16x8(make_uint4(pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3]), pack_bf16x2(t[4], t[5]),
                              pack_bf16x2(t[6], t[7])));
}

template <int HD, bool ALIBI, bool CAUSAL>
struct DqWave {
  f32x16 dq[HD / 32];  // dQ^T: lane holds query n, dims 32mb + 8(r/4) + 4hf + r%4
  bf16x8 qf[HD / 16];  // Q^T B operand (rotated), k-step s: dims 16s + 8hf .. +7
  bf16x8 df[HD / 16];  // dO^T B operand
  float lse2;          // this lane's query: log-sum-exp in log2 units
  float Dq;            // rowsum(dout * out)
  float c2, slope2;
  int qi, T, lane;
  int ktr[HD / 32];

  // One 64-key tile: K at kb (V swizzle), V at vb (K swizzle), in two halves
  // of 32 keys (a half's scores, dP and dS die before the next half starts).
  template <bool MASK>
  __device__ __forceinline__ void tile(LdsBytes kb, LdsBytes vb, int k0) {
    const int n = lane & 31, hf = lane >> 5;
    const int krow = perm_row(n);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int st = 0; st < HD / 16; ++st) {
        const bf16x8 ak = *reinterpret_cast<const LDS bf16x8*>(kb + v_off<HD>(32 * kb2 + krow, 2 * st + hf));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[st], s, 0, 0, 0);
        const bf16x8 avv = *reinterpret_cast<const LDS bf16x8*>(vb + k_off<HD>(32 * kb2 + krow, 2 * st + hf));
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(avv, df[st], dp, 0, 0, 0);
      }
      // register i is key k0 + 32 kb2 + 16(i/8) + 8hf + i%8
      const int dbase = k0 + 32 * kb2 + 8 * hf - qi;
      const float dbf = (float)dbase;
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float ci = (float)(16 * (i / 8) + (i % 8));
        float t;
        if constexpr (ALIBI) {
          const float bias = CAUSAL ? fmaf(slope2, ci, slope2 * dbf) : -slope2 * fabsf(dbf + ci);
          t = fmaf(s[i], c2, bias);
        } else {
          t = s[i] * c2;
        }
        if constexpr (MASK) {
          const int dk = dbase + 16 * (i / 8) + (i % 8);
          const bool vis = (dk + qi < T) && (!CAUSAL || dk <= 0);
          t = vis ? t : -INFINITY;
        }
        const float p = __builtin_amdgcn_exp2f(t - lse2);
        ds[i] = p * (dp[i] - Dq);
      }
      const bf16x8 d0 = pack8(ds), d1 = pack8(ds + 8);
#pragma unroll
      for (int mb = 0; mb < HD / 32; ++mb) {
        dq[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<HD>(kb, ktr[mb], 2 * kb2), d0, dq[mb], 0, 0, 0);
        dq[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<HD>(kb, ktr[mb], 2 * kb2 + 1), d1, dq[mb], 0, 0, 0);
      }
    }
  }
};

template <int HD, bool ALIBI, bool CAUSAL, bool GRAD_BF16>
__global__ __launch_bounds__(QT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_mfma_kernel(BwdArgs a, DqGrid gm) {
  using C = Cfg<HD>;
  // two stages (K with the V swizzle, then V with the K swizzle), each its own
  // LDS object so the DMA into one never makes the compiler wait before reads
  // of the other
  __shared__ __attribute__((aligned(16))) unsigned char s0[C::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char s1[C::STAGE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31, hf = lane >> 5;

  const int w = blockIdx.x;
  int unit, qrank;
  if (gm.xcd_aware) {
    const int upx = gm.units >> 3;
    const int j = w >> 3;
    unit = (w & 7) * upx + j % upx;
    qrank = j / upx;
  } else {
    unit = w % gm.units;
    qrank = w / gm.units;
  }
  const int qb = gm.nqb - 1 - qrank;
  const int hc = unit % gm.hchunks;
  const int pair = unit / gm.hchunks;
  const int kvh = pair % a.KV;
  const int b = pair / a.KV;
  const int head = kvh * a.group + hc * gm.hpw + (wave % gm.hpw);
  const int q0 = qb * gm.bm;
  const int qw0 = q0 + 32 * (wave / gm.hpw);
  const bool wave_active = qw0 < a.T;
  const long kvoff = ((long)b * a.KV + kvh) * (long)a.T * HD;
  const uint16_t* Kg = reinterpret_cast<const uint16_t*>(a.k) + kvoff;
  const uint16_t* Vg = reinterpret_cast<const uint16_t*>(a.v) + kvoff;
  const int q_last = min(a.T, q0 + gm.bm) - 1;
  const int nkt = CAUSAL ? (q_last / BN + 1) : (a.T + BN - 1) / BN;

  Dma<HD, QW, true, true> dma;
  dma.init(wave, lane);
  dma.issue(Kg, Vg, 0, a.T, s0, wave);

  DqWave<HD, ALIBI, CAUSAL> ws;
  ws.qi = qw0 + n;
  ws.T = a.T;
  ws.lane = lane;
  ws.c2 = a.scale * kLog2eM;
  ws.slope2 = ALIBI ? alibi_slope(a.alibi, head, a.H) * kLog2eM : 0.f;
  tr_offsets<HD>(lane, ws.ktr);
  const long row = ((long)b * a.H + head) * a.T + min(ws.qi, a.T - 1);
  {
    const uint4* qs = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) + row * HD);
    const uint4* gs = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.dout) + row * HD);
#pragma unroll
    for (int s = 0; s < HD / 16; ++s) {
      ws.qf[s] = as_bf16x8(qs[2 * s + hf]);
      ws.df[s] = as_bf16x8(gs[2 * s + hf]);
    }
    ws.lse2 = a.lse[row] * kLog2eM;
    ws.Dq = a.D[row];
  }
#pragma unroll
  for (int mb = 0; mb < HD / 32; ++mb) ws.dq[mb] = f32x16{};
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // tiles [0, kt_clean) are visible to every row of the workgroup
  const int kt_clean = min(nkt, CAUSAL ? min((q0 + 1) / BN, a.T / BN) : a.T / BN);
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  auto step = [&](int kt, auto mask_tag, auto par_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int P = decltype(par_tag)::value;
    unsigned char* cur = P ? s1 : s0;
    unsigned char* nxt = P ? s0 : s1;
    const int k0 = kt * BN;
    if (kt + 1 < nkt) dma.issue(Kg, Vg, kt + 1, a.T, nxt, wave);
    const bool run = wave_active && !(MASK && CAUSAL && k0 > qw0 + 31);
    if (run) ws.template tile<MASK>((LdsBytes)cur, (LdsBytes)(cur + C::K_BYTES), k0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  int kt = 0;
  for (; kt + 2 <= kt_clean; kt += 2) {
    step(kt, std::false_type{}, Even{});
    step(kt + 1, std::false_type{}, Odd{});
  }
  while (kt < nkt) {
    step(kt, std::true_type{}, Even{});
    if (++kt >= nkt) break;
    step(kt, std::true_type{}, Odd{});
    ++kt;
  }

  if (!wave_active || ws.qi >= a.T) return;
  // dq = R(-pos) scale dQ'^T: lane holds 4 consecutive dims per register group
  const int pos = a.pos0 + ws.qi;
#pragma unroll
  for (int mb = 0; mb < HD / 32; ++mb) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = 32 * mb + 8 * g4 + 4 * hf;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const float x0 = ws.dq[mb][4 * g4 + e] * a.scale, x1 = ws.dq[mb][4 * g4 + e + 1] * a.scale;
        float c = 1.f, sn = 0.f;
        if (a.rope) rope_cos_sin(pos, a.freqs.rev[(d + e) >> 1], c, sn);
        y[e] = rot0(x0, x1, c, -sn);
        y[e + 1] = rot1(x0, x1, c, -sn);
      }
      if constexpr (GRAD_BF16) {
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.dq) + row * HD + d) =
            make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.dq) + row * HD + d) = make_float4(y[0], y[1], y[2], y[3]);
      }
    }
  }
}

DqGrid make_dq_grid(const BwdArgs& a) {
  DqGrid gm;
  gm.hpw = (a.group % 4 == 0) ? 4 : (a.group % 2 == 0 ? 2 : 1);
  gm.hchunks = a.group / gm.hpw;
  gm.bm = 32 * (QW / gm.hpw);
  gm.nqb = (a.T + gm.bm - 1) / gm.bm;
  gm.units = a.B * a.KV * gm.hchunks;
  gm.xcd_aware = (gm.units % 8) == 0;
  return gm;
}

template <int HD, bool ALIBI, bool CAUSAL>
void launch_dq_g(const BwdArgs& a, hipStream_t s) {
  const DqGrid gm = make_dq_grid(a);
  const dim3 grid((unsigned)(gm.units * gm.nqb));
  if (a.grad_bf16) {
    hipLaunchKernelGGL((bwd_dq_mfma_kernel<HD, ALIBI, CAUSAL, true>), grid, dim3(QT), 0, s, a, gm);
  } else {
    hipLaunchKernelGGL((bwd_dq_mfma_kernel<HD, ALIBI, CAUSAL, false>), grid, dim3(QT), 0, s, a, gm);
  }
}

template <int HD>
void launch_dq_hd(const BwdArgs& a, hipStream_t s) {
  if (a.alibi) {
    if (a.causal) launch_dq_g<HD, true, true>(a, s);
    else launch_dq_g<HD, true, false>(a, s);
  } else {
    if (a.causal) launch_dq_g<HD, false, true>(a, s);
    else launch_dq_g<HD, false, false>(a, s);
  }
}

}  // namespace

bool bwd_mfma_supported(const BwdArgs& a) {
  if (!a.in_bf16 || !a.out_bf16 || (a.hd != 64 && a.hd != 128)) return false;
  if ((long)a.T * a.hd * 2 >= (1L << 31)) return false;  // buffer descriptors hold 32-bit sizes
  const DqGrid gm = make_dq_grid(a);
  return (long)gm.units * gm.nqb < (1L << 31);
}

hipError_t launch_bwd_dq_mfma(const BwdArgs& a, hipStream_t s) {
  if (a.hd == 128) {
    launch_dq_hd<128>(a, s);
  } else {
    launch_dq_hd<64>(a, s);
  }
  return hipGetLastError();
}

}  // namespace attn

namespace attn {

hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t s, const TimingHook& tm) {
  hipError_t e = tm.before(s);
  if (e != hipSuccess) return e;
  if ((e = launch_bwd_dq_mfma(a, s)) != hipSuccess) return e;
  if ((e = launch_bwd_dkv_valu(a, s)) != hipSuccess) return e;
  return tm.after(s);
}

}  // namespace attn
