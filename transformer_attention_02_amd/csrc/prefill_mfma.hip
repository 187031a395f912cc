// bf16 matrix-core prefill kernel for gfx950 (CDNA4).
//
// Computes the tiled online-softmax attention forward ("Building Grouped-Query
// Attention with RoPE and Flash Attention from Scratch", Step 3; recurrences of
// "Building a Transformer from Scratch", Part 3) with bf16 operands and fp32
// softmax statistics and accumulation (that page's mixed-precision roadmap item).
//
// Work decomposition
//   * A workgroup is 4 waves. It owns one block of query rows for up to 4 query
//     heads that share one key/value head (grouped-query packing), so every
//     K/V tile staged in LDS serves all of them.
//   * A wave owns 32 query rows of one head and computes S^T = K Q^T with
//     v_mfma_f32_32x32x16_bf16. In the 32x32 accumulator a lane holds one
//     query (column) and 16 keys (rows), so the row max and row sum are
//     in-lane reductions plus one exchange between the two half-waves.
//   * The key rows fed to the S^T contraction are permuted (bits 2 and 3 of
//     the row index swapped) so that accumulator registers 8u..8u+7 of a lane
//     hold 8 consecutive keys: the probabilities then feed O^T = V^T P^T as the
//     B operand straight from registers (rounded to bf16).
//   * K/V tiles of 64 keys are double-buffered in LDS: the global loads of tile
//     j+1 are in flight while tile j is computed. Both tiles are stored
//     row-major as loaded; V^T operands are read with ds_read_b64_tr_b16 (the
//     transposing LDS load of gfx950). XOR swizzles keep the operand reads free
//     of bank conflicts.
//   * Causal: tiles past the diagonal are never loaded; a wave skips tiles that
//     are entirely above its rows; only tiles crossing the diagonal (or the
//     ragged end of the sequence) are masked.
//   * Rotary embedding of Q is fused into the Q load (fp32 rotation, rounded to
//     bf16); K arrives already rotated (a pre-pass writes it once).
//   * Workgroups are numbered so that every workgroup touching one key/value
//     head lands on the same XCD (its L2 keeps that head's K/V), heaviest
//     causal blocks first.
#include "attn_internal.h"

namespace attn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 64;  // keys per tile
constexpr int NW = 4;   // waves per workgroup
constexpr int NT = NW * 64;

template <int HD>
struct Cfg {
  static constexpr int KCH = HD / 8;               // 16-byte chunks per key row
  static constexpr int K_BYTES = BN * HD * 2;      // K tile, row-major [key][hd]
  static constexpr int V_BYTES = BN * HD * 2;      // V tile, row-major [key][hd]
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int LOADS = BN * KCH / NT;      // 16-byte loads per thread per tensor
};

struct GridMap {
  int hpw;       // heads per workgroup (1, 2 or 4)
  int hchunks;   // group / hpw
  int bm;        // query rows per head per workgroup = 32 * (4 / hpw)
  int nqb;       // query blocks
  int units;     // B * KV * hchunks
  int xcd_aware;
};

// Byte offset of 16-byte chunk `c` of key row `r` in the K tile (XOR swizzle).
template <int HD>
__device__ __forceinline__ int k_off(int r, int c) {
  if constexpr (HD == 128) {
    return r * 256 + ((c ^ (r & 15)) << 4);
  } else {
    return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
  }
}

// Byte offset of 16-byte chunk `c` of key row `r` in the row-major V tile. The
// XOR spreads the 4-row x 64-byte blocks that one transposing load instruction
// touches (rows r..r+3, one 32-column slice) over all LDS banks.
template <int HD>
__device__ __forceinline__ int v_off(int r, int c) {
  if constexpr (HD == 128) {
    return r * 256 + ((c ^ ((r & 3) << 2)) << 4);
  } else {
    return r * 128 + ((c ^ (((r >> 1) & 1) << 2)) << 4);
  }
}

// Swap bits 2 and 3 of a row index in [0, 32).
__device__ __forceinline__ int perm_row(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Component i (a compile-time constant after unrolling) of a uint4, without taking its address.
__device__ __forceinline__ uint32_t comp(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ float xhalf(float x) { return __shfl_xor(x, 32); }

// Registers holding one K/V tile between its global load and its LDS store.
// Thread t moves chunks e = t + 256 i (key row e / KCH, 16-byte chunk e % KCH)
// of both tensors; every wave instruction covers whole rows, so the global
// loads are fully coalesced and the LDS stores are conflict-free.
template <int HD>
struct Stage {
  using C = Cfg<HD>;
  uint4 k[C::LOADS];
  uint4 v[C::LOADS];

  // Loads tile kt through buffer descriptors that start at the tile and end at
  // the slab end: rows at or past T read as zero.
  __device__ __forceinline__ void load(const uint16_t* Kg, const uint16_t* Vg, int kt, int T, int tid) {
    const int bytes = (T - kt * BN) * HD * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg + (long)kt * BN * HD, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg + (long)kt * BN * HD, bytes);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int e = tid + NT * i;  // row e / KCH, chunk e % KCH: byte offset 16 e
      k[i] = buffer_load16(rk, 16 * e);
      v[i] = buffer_load16(rv, 16 * e);
    }
  }

  __device__ __forceinline__ void store(unsigned char* kb, int tid) const {
    unsigned char* vb = kb + C::K_BYTES;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int e = tid + NT * i;
      const int r = e / C::KCH, c = e % C::KCH;
      *reinterpret_cast<uint4*>(kb + k_off<HD>(r, c)) = k[i];
      *reinterpret_cast<uint4*>(vb + v_off<HD>(r, c)) = v[i];
    }
  }
};

// One wave's online-softmax state over its 32 query rows, and the work of one
// 64-key tile. MASK selects the variant for tiles that cross the causal
// diagonal or the sequence end; every other tile runs without masking code.
template <int HD, bool ALIBI, bool CAUSAL>
struct WaveState {
  f32x16 oacc[HD / 32];  // O^T: lane holds query n, dims 32mb + 8(r/4) + 4hf + r%4
  bf16x8 qf[HD / 16];    // Q^T B operand, k-step s: dims 16s + 8hf .. +7
  float m_run;           // running max (log2 units), per row
  float l_run;           // this half-wave's part of the running denominator
  float c2;              // log2(e) / sqrt(hd)
  float slope2;          // ALiBi slope * log2(e)
  int qi;                // this lane's query row
  int T;
  int lane;

  template <bool MASK>
  __device__ __forceinline__ void tile(const unsigned char* kb, int k0) {
    using C = Cfg<HD>;
    const unsigned char* vb = kb + C::K_BYTES;
    const int n = lane & 31, hf = lane >> 5;
    // S^T = K Q^T; the K rows are read in permuted order (perm_row) so that
    // register i of the two accumulators holds key k0 + 32(i/16) + 16((i%16)/8) + 8hf + i%8.
    f32x16 sacc[2];
    const int krow = perm_row(n);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      sacc[kb2] = f32x16{};
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) {
        const uint4 av = *reinterpret_cast<const uint4*>(kb + k_off<HD>(32 * kb2 + krow, 2 * s + hf));
        sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), qf[s], sacc[kb2], 0, 0, 0);
      }
    }
    // Without ALiBi t keeps the raw scores (the max commutes with the positive
    // scale, which is folded into the exponent's FMA); with ALiBi t is the
    // scaled, biased score in log2 units.
    float t[32];
    const int dbase = k0 + 8 * hf - qi;  // key - query at register offset 0
    if constexpr (ALIBI) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float dk = (float)(dbase + 32 * (i / 16) + 16 * ((i % 16) / 8) + (i % 8));
        t[i] = fmaf(sacc[i / 16][i % 16], c2, slope2 * (CAUSAL ? dk : -fabsf(dk)));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) t[i] = sacc[i / 16][i % 16];
    }
    if constexpr (MASK) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int dk = dbase + 32 * (i / 16) + 16 * ((i % 16) / 8) + (i % 8);
        const bool vis = (dk + qi < T) && (!CAUSAL || dk <= 0);
        t[i] = vis ? t[i] : -INFINITY;
      }
    }
    float mx = t[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mx = fmaxf(mx, t[i]);
    mx = fmaxf(mx, xhalf(mx));
    const float ms = ALIBI ? mx : mx * c2;  // tile max in log2 units
    // Lazy rescale: a row's running max only moves when its tile max exceeds
    // it by more than 8 (a factor 2^8); otherwise the stale max is kept for
    // both the numerator and the denominator, which leaves O / l unchanged.
    // The decision is per row (a row that does not move multiplies by exactly
    // 1), so no row's arithmetic depends on another row's scores; the
    // wave-wide test only skips the multiplies when no row moves.
    const bool move = ms > m_run + 8.0f;
    if (__any(move)) {
      // (a side effect keeps this a real branch: the compiler would otherwise
      // hoist the multiplies, which are an identity when no row moves)
      asm volatile("; rescale" ::: "memory");
      const float alpha = move ? __builtin_amdgcn_exp2f(m_run - ms) : 1.0f;
      m_run = move ? ms : m_run;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < HD / 32; ++mb) oacc[mb] *= alpha;
    }
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      t[i] = __builtin_amdgcn_exp2f(ALIBI ? t[i] - m_run : fmaf(t[i], c2, -m_run));
      lsum += t[i];
    }
    l_run += lsum;
    // O^T += V^T P^T over four 16-key steps. P^T (the B operand) comes straight
    // from t[8u .. 8u+7]; V^T is read with transposing loads: source lane i of a
    // 16-lane group points at key row 16u + 8hf + i/4 (+4), columns d0 + 4(i%4),
    // and lane i then holds V[those 4 keys][d0 + i].
    const int li = lane & 15;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 pw = make_uint4(pack_bf16x2(t[8 * u + 0], t[8 * u + 1]), pack_bf16x2(t[8 * u + 2], t[8 * u + 3]),
                                  pack_bf16x2(t[8 * u + 4], t[8 * u + 5]), pack_bf16x2(t[8 * u + 6], t[8 * u + 7]));
      const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
      for (int mb = 0; mb < HD / 32; ++mb) {
        const int col = 32 * mb + 16 * ((lane >> 4) & 1) + 4 * (li & 3);
        const int r = 16 * u + 8 * hf + (li >> 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vb + v_off<HD>(r, col >> 3) + (col & 7) * 2));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vb + v_off<HD>(r + 4, col >> 3) + (col & 7) * 2));
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, oacc[mb], 0, 0, 0);
      }
    }
  }
};

template <int HD, bool ALIBI, bool CAUSAL, bool OUT_BF16>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_mfma_kernel(PrefillArgs a, GridMap gm) {
  using C = Cfg<HD>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;

  // ---- workgroup -> (unit = (b, kv head, head chunk), query block), heavy blocks first
  const int w = blockIdx.x;
  int unit, qrank;
  if (gm.xcd_aware) {
    // Consecutive workgroups go round-robin to the 8 XCDs. XCD x owns units
    // [x*upx, (x+1)*upx) and interleaves them, heaviest query blocks first.
    // (Working through one unit at a time measured slower: all of an XCD's
    // workgroups then hit the same K/V lines at once.)
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

  // The first K/V tile's global loads are in flight during the Q set-up.
  Stage<HD> st;
  st.load(Kg, Vg, 0, a.T, tid);

  WaveState<HD, ALIBI, CAUSAL> ws;
  ws.qi = qw0 + n;
  ws.T = a.T;
  ws.lane = lane;
  ws.c2 = a.scale_log2;
  ws.slope2 = ALIBI ? alibi_slope(a.alibi, head, a.H) * 1.4426950408889634f : 0.f;
  ws.m_run = -INFINITY;
  ws.l_run = 0.f;
#pragma unroll
  for (int mb = 0; mb < HD / 32; ++mb) ws.oacc[mb] = f32x16{};

  // ---- Q rows -> B operand (rotated in fp32, rounded to bf16). The rotary
  // cos/sin of the workgroup's bm rows are computed once into LDS (layout
  // [pair][row], so lanes reading consecutive rows hit distinct banks) and
  // shared by the waves of all heads in the workgroup.
  {
    const int qrow = min(ws.qi, a.T - 1);
    const uint4* src =
        reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) + (((long)b * a.H + head) * a.T + qrow) * HD);
    uint4 qraw[HD / 16];
#pragma unroll
    for (int s = 0; s < HD / 16; ++s) qraw[s] = src[2 * s + hf];
    if (a.rope) {
      float2* cs = reinterpret_cast<float2*>(smem);  // [HD/2][bm]
      for (int e = tid; e < (HD / 2) * gm.bm; e += NT) {
        const int r = e % gm.bm, p = e / gm.bm;
        float c, sn;
        rope_cos_sin(a.pos0 + q0 + r, a.freqs.rev[p], c, sn);
        cs[e] = make_float2(c, sn);
      }
      __syncthreads();
      const int r = ws.qi - q0;
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) {
        uint32_t d[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float2 t = cs[(8 * s + 4 * hf + p) * gm.bm + r];
          const uint32_t x = comp(qraw[s], p);
          const float x0 = bf16_bits_to_f32(x & 0xffffu), x1 = bf16_bits_to_f32(x >> 16);
          d[p] = pack_bf16x2(x0 * t.x - x1 * t.y, x0 * t.y + x1 * t.x);
        }
        ws.qf[s] = as_bf16x8(make_uint4(d[0], d[1], d[2], d[3]));
      }
      __syncthreads();  // the table area is reused by the K/V tiles
    } else {
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) ws.qf[s] = as_bf16x8(qraw[s]);
    }
  }

  st.store(smem, tid);
  __syncthreads();

  // Tiles [0, kt_clean) need no mask for any row of the workgroup: every key is
  // at or before the first query row (causal) and inside the sequence.
  const int kt_clean = min(nkt, CAUSAL ? min((q0 + 1) / BN, a.T / BN) : a.T / BN);
  int kt = 0;
  for (; kt < kt_clean; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nkt) st.load(Kg, Vg, kt + 1, a.T, tid);
    if (wave_active) ws.template tile<false>(smem + stage * C::STAGE, kt * BN);
    if (kt + 1 < nkt) st.store(smem + (stage ^ 1) * C::STAGE, tid);
    __syncthreads();
  }
  for (; kt < nkt; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nkt) st.load(Kg, Vg, kt + 1, a.T, tid);
    const int k0 = kt * BN;
    if (wave_active && !(CAUSAL && k0 > qw0 + 31)) ws.template tile<true>(smem + stage * C::STAGE, k0);
    if (kt + 1 < nkt) st.store(smem + (stage ^ 1) * C::STAGE, tid);
    __syncthreads();
  }

  if (!wave_active) return;
  const float l_tot = ws.l_run + xhalf(ws.l_run);
  const int qi = ws.qi;
  if (qi >= a.T) return;
  const float inv_l = 1.0f / l_tot;
  const long orow = (((long)b * a.H + head) * a.T + qi) * HD;
#pragma unroll
  for (int mb = 0; mb < HD / 32; ++mb) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = 32 * mb + 8 * g4 + 4 * hf;
      const float o0 = ws.oacc[mb][4 * g4 + 0] * inv_l, o1 = ws.oacc[mb][4 * g4 + 1] * inv_l;
      const float o2 = ws.oacc[mb][4 * g4 + 2] * inv_l, o3 = ws.oacc[mb][4 * g4 + 3] * inv_l;
      if constexpr (OUT_BF16) {
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + orow + d) =
            make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + orow + d) = make_float4(o0, o1, o2, o3);
      }
    }
  }
  if (a.lse && hf == 0) a.lse[((long)b * a.H + head) * a.T + qi] = (ws.m_run + log2f(l_tot)) * 0.69314718055994531f;
}

GridMap make_grid(const PrefillArgs& a) {
  GridMap gm;
  gm.hpw = (a.group % 4 == 0) ? 4 : (a.group % 2 == 0 ? 2 : 1);
  gm.hchunks = a.group / gm.hpw;
  gm.bm = 32 * (NW / gm.hpw);
  gm.nqb = (a.T + gm.bm - 1) / gm.bm;
  gm.units = a.B * a.KV * gm.hchunks;
  gm.xcd_aware = (gm.units % 8) == 0;
  return gm;
}

template <int HD, bool ALIBI, bool CAUSAL>
void launch_out(const PrefillArgs& a, const GridMap& gm, dim3 grid, hipStream_t s) {
  if (a.out_bf16) {
    hipLaunchKernelGGL((prefill_mfma_kernel<HD, ALIBI, CAUSAL, true>), grid, dim3(NT), 0, s, a, gm);
  } else {
    hipLaunchKernelGGL((prefill_mfma_kernel<HD, ALIBI, CAUSAL, false>), grid, dim3(NT), 0, s, a, gm);
  }
}

template <int HD>
void launch_hd(const PrefillArgs& a, const GridMap& gm, dim3 grid, hipStream_t s) {
  if (a.alibi) {
    if (a.causal) launch_out<HD, true, true>(a, gm, grid, s);
    else launch_out<HD, true, false>(a, gm, grid, s);
  } else {
    if (a.causal) launch_out<HD, false, true>(a, gm, grid, s);
    else launch_out<HD, false, false>(a, gm, grid, s);
  }
}

}  // namespace

bool prefill_mfma_supported(const PrefillArgs& a, int bf16) {
  if (!bf16 || (a.hd != 64 && a.hd != 128)) return false;
  if ((long)a.T * a.hd * 2 >= (1L << 31)) return false;  // buffer descriptors hold 32-bit sizes
  const GridMap gm = make_grid(a);
  return (long)gm.units * gm.nqb < (1L << 31);
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s) {
  const GridMap gm = make_grid(a);
  const dim3 grid((unsigned)(gm.units * gm.nqb));
  if (a.hd == 128) {
    launch_hd<128>(a, gm, grid, s);
  } else {
    launch_hd<64>(a, gm, grid, s);
  }
  return hipGetLastError();
}

}  // namespace attn
