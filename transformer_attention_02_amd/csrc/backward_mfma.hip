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
    int o = kt_off<HD>(8 * hf + (li >> 2), col >> 3) + (col & 7) * 2;
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(o));
#endif
    off[mb] = o;
  }
}

// A^T operand of 16 rows (16u .. 16u+15 of the tile) x 32 columns (block mb)
// read transposed: lane i of a 16-lane group receives column d0 + i of 4 rows
// per 8-byte load; the second load is 4 rows down (K-tile swizzle).
template <int HD>
__device__ __forceinline__ bf16x8 read_tr(LdsBytes base, int off, int u) {
  LdsBytes p = base + off + 16 * u * HD * 2;
  LdsBytes p2 = base + (off ^ kt_xor4<HD>()) + (16 * u + 4) * HD * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)p2);
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

  // One 64-key tile: K at kb (K-tile swizzle), V at vb (K swizzle), in two halves
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
        const bf16x8 ak = *reinterpret_cast<const LDS bf16x8*>(kb + kt_off<HD>(32 * kb2 + krow, 2 * st + hf));
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
  // two stages (K with the K-tile swizzle, then V with the K swizzle), each its own
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

  Dma<HD, QW, SWZ_KT, SWZ_K> dma;
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
    const uint4* os = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.out) + row * HD);
    // D = <dout, out> of this lane's query: each half of the lane pair (n,
    // n + 32) holds every other 8-dim chunk of the row
    float dsum = 0.f;
#pragma unroll
    for (int s = 0; s < HD / 16; ++s) {
      ws.qf[s] = as_bf16x8(qs[2 * s + hf]);
      const uint4 gv = gs[2 * s + hf], ov = os[2 * s + hf];
      ws.df[s] = as_bf16x8(gv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t gw = comp(gv, e), ow = comp(ov, e);
        dsum = fmaf(__uint_as_float(gw << 16), __uint_as_float(ow << 16), dsum);
        dsum = fmaf(__uint_as_float(gw & 0xffff0000u), __uint_as_float(ow & 0xffff0000u), dsum);
      }
    }
    ws.Dq = dsum + __shfl_xor(dsum, 32);
    ws.lse2 = a.lse[row] * kLog2eM;
    // the dk/dv kernel reads D of every row
    if (hf == 0 && wave_active && ws.qi < a.T) a.D[row] = ws.Dq;
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

// --------------------------------------------------------------- dk/dv kernel
// 16 keys per wave on v_mfma_f32_16x16x32_bf16, so that a wave's state (dK'^T
// and dV^T for its keys, their K'/V operands) stays near 100 registers and two
// waves share each SIMD.
constexpr int KW = 8;        // waves per dk/dv workgroup
constexpr int KT = KW * 64;
constexpr int KB = 16 * KW;  // keys per workgroup

struct DkvGrid {
  int nkb;    // key blocks of KB keys
  int units;  // B * KV
  int xcd_aware;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Transposing read of a 16x32 A operand (16 columns of the tile: one 16-dim
// block; 32 rows: queries 8g .. 8g+7 of each 16-lane group g, four per load).
__device__ __forceinline__ bf16x8 read_tr32(LdsBytes p, int second) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(p + second));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int HD, bool ALIBI, bool CAUSAL>
struct DkvWave {
  f32x4 dk[HD / 16];   // dK'^T block b: lane holds key l%16, dims 16b + 4g + i
  f32x4 dv[HD / 16];   // dV^T, same layout
  bf16x8 kf[HD / 32];  // K'^T B operand, k-step s: dims 32s + 8g .. +7 of key l%16
  bf16x8 vf[HD / 32];  // V^T B operand
  float c2, slope2;
  int kk, kw0, T, lane;
  int rbase;             // byte offset of this lane's operand row (chunk part excluded)
  int rsw;               // its swizzle
  int tro[HD / 16];      // transposing-read offsets, one per 16-dim block

  __device__ __forceinline__ void init_offsets() {
    const int l16 = lane & 15, g = lane >> 4;
    // S / dP rows: query 8(l16/4) + l16%4 of each 32-query chunk (+4 for the
    // second 16-row block), so that block 0 / 1 registers hold queries
    // 8g .. 8g+3 / 8g+4 .. 8g+7 of the chunk: the B operand of dV^T, dK'^T
    const int r = 8 * (l16 >> 2) + (l16 & 3);
    rbase = r * HD * 2;
    rsw = q_swz<HD>(r);
    const int rt = 8 * g + (l16 >> 2);
#pragma unroll
    for (int bb = 0; bb < HD / 16; ++bb) {
      const int col = 16 * bb + 4 * (l16 & 3);
      int o = q_off<HD>(rt, col >> 3) + (col & 7) * 2;
#if defined(__HIP_DEVICE_COMPILE__)
      asm volatile("" : "+v"(o));
#endif
      tro[bb] = o;
    }
  }

  // One 64-row query tile starting at query q0: Q' at qb and dO at gb (query
  // swizzle), the rows' lse and D at lb / db (64 floats each). Operand reads
  // run a few ahead of the matrix-core instructions that consume them
  // (scheduling groups), so LDS latency hides behind the MFMA chain.
  template <bool MASK>
  __device__ __forceinline__ void tile(LdsBytes qb, LdsBytes gb, LdsBytes lb, LdsBytes db, int q0) {
    constexpr int NS = HD / 32;  // k-steps of the S / dP contractions
    constexpr int NB = HD / 16;  // 16-dim blocks of dK'^T / dV^T
    const int g = lane >> 4;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // (causal) every query of the chunk precedes every key of the wave
      if (MASK && CAUSAL && q0 + 32 * c + 31 < kw0) continue;
      // S = Q' K'^T and dP = dO V^T for the chunk's two 16-row blocks
      bf16x8 oq[2][NS], og[2][NS];
#pragma unroll
      for (int st = 0; st < NS; ++st)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int o = rbase + (32 * c + 4 * b) * HD * 2 + (((4 * st + g) ^ rsw) << 4);
          oq[b][st] = *reinterpret_cast<const LDS bf16x8*>(qb + o);
          og[b][st] = *reinterpret_cast<const LDS bf16x8*>(gb + o);
        }
      const int r0 = 32 * c + 8 * g;
      const f32x4 la = *reinterpret_cast<const LDS f32x4*>(lb + 4 * r0);
      const f32x4 lc = *reinterpret_cast<const LDS f32x4*>(lb + 4 * r0 + 16);
      const f32x4 da = *reinterpret_cast<const LDS f32x4*>(db + 4 * r0);
      const f32x4 dc = *reinterpret_cast<const LDS f32x4*>(db + 4 * r0 + 16);
      f32x4 s[2] = {f32x4{}, f32x4{}}, dp[2] = {f32x4{}, f32x4{}};
#pragma unroll
      for (int st = 0; st < NS; ++st)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          s[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oq[b][st], kf[st], s[b], 0, 0, 0);
          dp[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(og[b][st], vf[st], dp[b], 0, 0, 0);
        }
      // 4 reads ahead, then one read per MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 4 * NS - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // lse and D
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

      // From here to the chunk's last MFMA the wave runs its exp / dS work and
      // the products that consume it at raised issue priority, ahead of a wave
      // starting its S / dP products (measured: the backward call ~2% faster).
      __builtin_amdgcn_s_setprio(1);
      // register i of block b is query q0 + 32c + 8g + 4b + i
      const int dbase = kk - (q0 + r0);  // key - query at j = 0
      const float dbf = (float)dbase;
      float p[8], ds[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float sv = s[j / 4][j % 4], dpv = dp[j / 4][j % 4];
        const float lse = j < 4 ? la[j] : lc[j - 4];
        const float dd = j < 4 ? da[j] : dc[j - 4];
        float t;
        if constexpr (ALIBI) {
          const float bias = CAUSAL ? fmaf(-slope2, (float)j, slope2 * dbf) : -slope2 * fabsf(dbf - (float)j);
          t = fmaf(sv, c2, bias);
        } else {
          t = sv * c2;
        }
        if constexpr (MASK) {
          const bool vis = (q0 + r0 + j < T) && (!CAUSAL || dbase <= j);
          t = vis ? t : -INFINITY;
        }
        p[j] = __builtin_amdgcn_exp2f(fmaf(lse, -kLog2eM, t));
        ds[j] = p[j] * (dpv - dd);
      }
      const bf16x8 pb = pack8(p), dsb = pack8(ds);
      // dV^T += dO^T P and dK'^T += Q'^T dS, one 16-dim block at a time
      bf16x8 tg[NB], tq[NB];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const int o = tro[bb] + 32 * c * HD * 2;
        tg[bb] = read_tr32(gb + o, 4 * HD * 2);
        tq[bb] = read_tr32(qb + o, 4 * HD * 2);
      }
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        dv[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tg[bb], pb, dv[bb], 0, 0, 0);
        dk[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tq[bb], dsb, dk[bb], 0, 0, 0);
      }
      // 8 transposing reads (4 operands) ahead, then two per MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 2 * NB - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_s_setprio(0);
    }
  }
};

// 64 floats of one row vector (lse or D) straight into LDS; rows at or past
// `rows` read as zero.
__device__ __forceinline__ void dma_row64(const float* g, int rows, unsigned char* dst, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = make_rsrc(g, rows * 4);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)dst, 4, 4 * lane, 0, 0, 0);
#endif
}

template <int HD, bool ALIBI, bool CAUSAL, bool GRAD_BF16>
__global__ __launch_bounds__(KT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkv_mfma_kernel(BwdArgs a, DkvGrid gm) {
  using C = Cfg<HD>;
  constexpr int SB = C::STAGE + 512;  // Q' tile, dO tile, 64 lse, 64 D
  __shared__ __attribute__((aligned(16))) unsigned char s0[SB];
  __shared__ __attribute__((aligned(16))) unsigned char s1[SB];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4;

  // The key blocks of one (batch, KV head) run side by side on one XCD,
  // heaviest (earliest, under the causal mask) first, and all of them stream
  // the query tiles in the same order, so each tile is fetched into that XCD's
  // L2 once for all of them.
  const int w = blockIdx.x;
  int unit, kblk;
  if (gm.xcd_aware) {
    const int upx = gm.units >> 3;
    const int j = w >> 3;
    unit = (w & 7) * upx + j / gm.nkb;
    kblk = j % gm.nkb;
  } else {
    unit = w / gm.nkb;
    kblk = w % gm.nkb;
  }
  const int kvh = unit % a.KV;
  const int b = unit / a.KV;
  const int kb0 = kblk * KB;
  const int qt_lo = CAUSAL ? kb0 / BN : 0;
  const int nqt = (a.T + BN - 1) / BN;
  const int nq = nqt - qt_lo;
  const int total = a.group * nq;

  Dma<HD, KW, SWZ_Q, SWZ_Q> dma;
  dma.init(wave, lane);
  // tile idx: query tile nqt-1-idx/group (last first) of head idx%group
  auto issue = [&](int idx, unsigned char* stage) __attribute__((always_inline)) {
    const int hh = idx % a.group, qt = nqt - 1 - idx / a.group;
    const long hrow = ((long)b * a.H + kvh * a.group + hh) * a.T;
    dma.issue(reinterpret_cast<const uint16_t*>(a.q) + hrow * HD, reinterpret_cast<const uint16_t*>(a.dout) + hrow * HD,
              qt, a.T, stage, wave);
    if (wave == 0) dma_row64(a.lse + hrow + qt * BN, a.T - qt * BN, stage + C::STAGE, lane);
    if (wave == 1) dma_row64(a.D + hrow + qt * BN, a.T - qt * BN, stage + C::STAGE + 256, lane);
  };
  issue(0, s0);

  DkvWave<HD, ALIBI, CAUSAL> ws;
  ws.kw0 = kb0 + 16 * wave;
  ws.kk = ws.kw0 + (lane & 15);
  ws.T = a.T;
  ws.lane = lane;
  ws.c2 = a.scale * kLog2eM;
  ws.slope2 = 0.f;  // per query head: set for each tile
  ws.init_offsets();
  const long krow = ((long)b * a.KV + kvh) * a.T + min(ws.kk, a.T - 1);
  {
    const uint4* ks = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.k) + krow * HD);
    const uint4* vs = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.v) + krow * HD);
#pragma unroll
    for (int st = 0; st < HD / 32; ++st) {
      ws.kf[st] = as_bf16x8(ks[4 * st + g]);
      ws.vf[st] = as_bf16x8(vs[4 * st + g]);
    }
  }
#pragma unroll
  for (int bb = 0; bb < HD / 16; ++bb) ws.dk[bb] = ws.dv[bb] = f32x4{};
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  auto step = [&](int idx, auto mask_tag, auto par_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int P = decltype(par_tag)::value;
    unsigned char* cur = P ? s1 : s0;
    unsigned char* nxt = P ? s0 : s1;
    if (idx + 1 < total) issue(idx + 1, nxt);
    const int q0 = (nqt - 1 - idx / a.group) * BN;
    if constexpr (ALIBI) ws.slope2 = alibi_slope(a.alibi, kvh * a.group + idx % a.group, a.H) * kLog2eM;
    ws.template tile<MASK>((LdsBytes)cur, (LdsBytes)(cur + C::K_BYTES), (LdsBytes)(cur + C::STAGE),
                           (LdsBytes)(cur + C::STAGE + 256), q0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // a tile needs the mask when it reaches the diagonal of the key block or
  // the end of the sequence
  auto masked = [&](int idx) __attribute__((always_inline)) {
    const int q0 = (nqt - 1 - idx / a.group) * BN;
    return (CAUSAL && q0 < kb0 + KB) || q0 + BN > a.T;
  };
  for (int idx = 0; idx < total; idx += 2) {
    if (masked(idx)) step(idx, std::true_type{}, Even{});
    else step(idx, std::false_type{}, Even{});
    if (idx + 1 >= total) break;
    if (masked(idx + 1)) step(idx + 1, std::true_type{}, Odd{});
    else step(idx + 1, std::false_type{}, Odd{});
  }

  if (ws.kk >= a.T) return;
  const int pos = a.pos0 + ws.kk;
#pragma unroll
  for (int bb = 0; bb < HD / 16; ++bb) {
    const int d = 16 * bb + 4 * g;
    float y[4], z[4];
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const float x0 = ws.dk[bb][e] * a.scale, x1 = ws.dk[bb][e + 1] * a.scale;
      float c = 1.f, sn = 0.f;
      if (a.rope) rope_cos_sin(pos, a.freqs.rev[(d + e) >> 1], c, sn);
      y[e] = rot0(x0, x1, c, -sn);
      y[e + 1] = rot1(x0, x1, c, -sn);
      z[e] = ws.dv[bb][e];
      z[e + 1] = ws.dv[bb][e + 1];
    }
    const long o = krow * HD + d;
    if constexpr (GRAD_BF16) {
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.dk) + o) =
          make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.dv) + o) =
          make_uint2(pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3]));
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.dk) + o) = make_float4(y[0], y[1], y[2], y[3]);
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.dv) + o) = make_float4(z[0], z[1], z[2], z[3]);
    }
  }
}

DkvGrid make_dkv_grid(const BwdArgs& a) {
  DkvGrid gm;
  gm.nkb = (a.T + KB - 1) / KB;
  gm.units = a.B * a.KV;
  gm.xcd_aware = (gm.units % 8) == 0;
  return gm;
}

template <int HD, bool ALIBI, bool CAUSAL>
void launch_dkv_g(const BwdArgs& a, hipStream_t s) {
  const DkvGrid gm = make_dkv_grid(a);
  const dim3 grid((unsigned)(gm.units * gm.nkb));
  if (a.grad_bf16) {
    hipLaunchKernelGGL((bwd_dkv_mfma_kernel<HD, ALIBI, CAUSAL, true>), grid, dim3(KT), 0, s, a, gm);
  } else {
    hipLaunchKernelGGL((bwd_dkv_mfma_kernel<HD, ALIBI, CAUSAL, false>), grid, dim3(KT), 0, s, a, gm);
  }
}

template <int HD>
void launch_dkv_hd(const BwdArgs& a, hipStream_t s) {
  if (a.alibi) {
    if (a.causal) launch_dkv_g<HD, true, true>(a, s);
    else launch_dkv_g<HD, true, false>(a, s);
  } else {
    if (a.causal) launch_dkv_g<HD, false, true>(a, s);
    else launch_dkv_g<HD, false, false>(a, s);
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

hipError_t launch_bwd_dkv_mfma(const BwdArgs& a, hipStream_t s) {
  if (a.hd == 128) {
    launch_dkv_hd<128>(a, s);
  } else {
    launch_dkv_hd<64>(a, s);
  }
  return hipGetLastError();
}

}  // namespace attn

namespace attn {

hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t s, const TimingHook& tm) {
  hipError_t e = tm.before(s);
  if (e != hipSuccess) return e;
  if ((e = launch_bwd_dq_mfma(a, s)) != hipSuccess) return e;
  if ((e = launch_bwd_dkv_mfma(a, s)) != hipSuccess) return e;
  return tm.after(s);
}

}  // namespace attn
