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
//     transposing LDS load of gfx950). Padded row pitches keep the operand
//     reads free of bank conflicts.
//   * Causal: tiles past the diagonal are never loaded; a wave skips tiles that
//     are entirely above its rows; only tiles crossing the diagonal (or the
//     ragged end of the sequence) are masked.
//   * Rotary embedding of Q is fused into the Q load (fp32 rotation, rounded to
//     bf16); K arrives already rotated (a pre-pass writes it once).
//   * Workgroups are numbered so that every workgroup touching one key/value
//     head lands on the same XCD (its L2 keeps that head's K/V), heaviest
//     causal blocks first.
#include <type_traits>

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
  // Padded row pitches keep every MFMA operand read free of LDS bank conflicts
  // while leaving the addresses affine (a per-lane base plus immediates):
  //  * K rows (pitch 2hd + 16): the 16 lanes of a ds_read_b128 read one 16-byte
  //    chunk of 16 different rows, which land on 16 disjoint 4-bank groups;
  //  * V rows (pitch 2hd + 64): a transposing load reads 4 consecutive rows x
  //    32 bytes per 16-lane group (64 bytes for the 32 lanes served together),
  //    and the 64-byte skew puts the 4 rows on disjoint bank ranges.
  static constexpr int KP = HD * 2 + 16;
  static constexpr int VP = HD * 2 + 64;
  static constexpr int K_BYTES = BN * KP;          // K tile, row-major [key][hd]
  static constexpr int V_BYTES = BN * VP;          // V tile, row-major [key][hd]
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int LOADS = BN * KCH / NT;      // 16-byte loads per thread per tensor
};

struct GridMap {
  int hpw;       // heads per workgroup (1, 2 or 4)
  int hchunks;   // group / hpw
  int bm;        // query rows per head per workgroup = 32 * QB * (4 / hpw)
  int nqb;       // query blocks
  int units;     // B * KV * hchunks
  int xcd_aware;
};

// Byte offset of 16-byte chunk `c` of key row `r` in the K / V tile.
template <int HD>
__device__ __forceinline__ int k_off(int r, int c) { return r * Cfg<HD>::KP + c * 16; }
template <int HD>
__device__ __forceinline__ int v_off(int r, int c) { return r * Cfg<HD>::VP + c * 16; }

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

// One wave's online-softmax state over QB blocks of 32 query rows (rows qi + 32j
// for block j), and the work of one 64-key tile. Each K and V operand read from
// LDS feeds the MFMAs of all QB blocks. MASK selects the variant for tiles that
// cross the causal diagonal or the sequence end; every other tile runs without
// masking code.
template <int HD, bool ALIBI, bool CAUSAL, int QB>
struct WaveState {
  f32x16 oacc[QB][HD / 32];  // O^T: lane holds query n, dims 32mb + 8(r/4) + 4hf + r%4
  bf16x8 qf[QB][HD / 16];    // Q^T B operand, k-step s: dims 16s + 8hf .. +7
  float m_run[QB];           // running max (log2 units), per row
  float l_run[QB];           // this half-wave's part of the running denominator
  float c2;                  // log2(e) / sqrt(hd)
  float slope2;              // ALiBi slope * log2(e)
  int qi;                    // this lane's query row in block 0
  int T;
  int lane;

  template <bool MASK>
  __device__ __forceinline__ void tile(const unsigned char* kb, int k0) {
    using C = Cfg<HD>;
    const unsigned char* vb = kb + C::K_BYTES;
    const int n = lane & 31, hf = lane >> 5;
    // S^T = K Q^T; the K rows are read in permuted order (perm_row) so that
    // register i of the two accumulators holds key k0 + 32(i/16) + 16((i%16)/8) + 8hf + i%8.
    f32x16 sacc[QB][2];
    const int krow = perm_row(n);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int j = 0; j < QB; ++j) sacc[j][kb2] = f32x16{};
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) {
        const bf16x8 av = as_bf16x8(*reinterpret_cast<const uint4*>(kb + k_off<HD>(32 * kb2 + krow, 2 * s + hf)));
#pragma unroll
        for (int j = 0; j < QB; ++j)
          sacc[j][kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[j][s], sacc[j][kb2], 0, 0, 0);
      }
    }
    bf16x8 pb[QB][4];
    bool live[QB];
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const int qj = qi + 32 * j;
      // a block whose rows all precede the tile's first key contributes nothing
      live[j] = !(MASK && CAUSAL && k0 > (qi - n) + 32 * j + 31);
      if (!live[j]) continue;
      // Without ALiBi t keeps the raw scores (the max commutes with the positive
      // scale, which is folded into the exponent's FMA); with ALiBi t is the
      // scaled, biased score in log2 units.
      float t[32];
      const int dbase = k0 + 8 * hf - qj;  // key - query at register offset 0
      if constexpr (ALIBI) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const float dk = (float)(dbase + 32 * (i / 16) + 16 * ((i % 16) / 8) + (i % 8));
          t[i] = fmaf(sacc[j][i / 16][i % 16], c2, slope2 * (CAUSAL ? dk : -fabsf(dk)));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) t[i] = sacc[j][i / 16][i % 16];
      }
      if constexpr (MASK) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int dk = dbase + 32 * (i / 16) + 16 * ((i % 16) / 8) + (i % 8);
          const bool vis = (dk + qj < T) && (!CAUSAL || dk <= 0);
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
      const bool move = ms > m_run[j] + 8.0f;
      if (__any(move)) {
        // (a side effect keeps this a real branch: the compiler would otherwise
        // hoist the multiplies, which are an identity when no row moves)
        asm volatile("; rescale" ::: "memory");
        const float alpha = move ? __builtin_amdgcn_exp2f(m_run[j] - ms) : 1.0f;
        m_run[j] = move ? ms : m_run[j];
        l_run[j] *= alpha;
#pragma unroll
        for (int mb = 0; mb < HD / 32; ++mb) oacc[j][mb] *= alpha;
      }
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        t[i] = __builtin_amdgcn_exp2f(ALIBI ? t[i] - m_run[j] : fmaf(t[i], c2, -m_run[j]));
        lsum += t[i];
      }
      l_run[j] += lsum;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        pb[j][u] = as_bf16x8(make_uint4(pack_bf16x2(t[8 * u + 0], t[8 * u + 1]), pack_bf16x2(t[8 * u + 2], t[8 * u + 3]),
                                        pack_bf16x2(t[8 * u + 4], t[8 * u + 5]), pack_bf16x2(t[8 * u + 6], t[8 * u + 7])));
    }
    // O^T += V^T P^T over four 16-key steps. P^T (the B operand) comes straight
    // from the probabilities; V^T is read with transposing loads: source lane i
    // of a 16-lane group points at key row 16u + 8hf + i/4 (+4), columns
    // d0 + 4(i%4), and lane i then holds V[those 4 keys][d0 + i].
    const int li = lane & 15;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int mb = 0; mb < HD / 32; ++mb) {
        const int col = 32 * mb + 16 * ((lane >> 4) & 1) + 4 * (li & 3);
        const int r = 16 * u + 8 * hf + (li >> 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vb + v_off<HD>(r, col >> 3) + (col & 7) * 2));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vb + v_off<HD>(r + 4, col >> 3) + (col & 7) * 2));
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int j = 0; j < QB; ++j)
          if (live[j]) oacc[j][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[j][u], oacc[j][mb], 0, 0, 0);
      }
    }
  }
};

// QB = query blocks of 32 rows per wave. QB = 2: one wave per SIMD (the state
// needs ~400 VGPRs) and a 3-stage LDS ring, so tile t+2 is in flight while tile
// t is computed. QB = 1: two waves per SIMD and a double buffer.
template <int QB>
struct Sched {
  static constexpr int STAGES = QB == 2 ? 3 : 2;
  static constexpr int WAVES_PER_EU = QB == 2 ? 1 : 2;
};

template <int HD, bool ALIBI, bool CAUSAL, bool OUT_BF16, int QB>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(Sched<QB>::WAVES_PER_EU, Sched<QB>::WAVES_PER_EU)))
void prefill_mfma_kernel(PrefillArgs a, GridMap gm) {
  using C = Cfg<HD>;
  constexpr int STAGES = Sched<QB>::STAGES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[STAGES * C::STAGE];

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
  const int qw0 = q0 + 32 * QB * (wave / gm.hpw);
  const bool wave_active = qw0 < a.T;

  const long kvoff = ((long)b * a.KV + kvh) * (long)a.T * HD;
  const uint16_t* Kg = reinterpret_cast<const uint16_t*>(a.k) + kvoff;
  const uint16_t* Vg = reinterpret_cast<const uint16_t*>(a.v) + kvoff;
  const int q_last = min(a.T, q0 + gm.bm) - 1;
  const int nkt = CAUSAL ? (q_last / BN + 1) : (a.T + BN - 1) / BN;

  // The first K/V tile's global loads are in flight during the Q set-up.
  Stage<HD> st;
  st.load(Kg, Vg, 0, a.T, tid);

  WaveState<HD, ALIBI, CAUSAL, QB> ws;
  ws.qi = qw0 + n;
  ws.T = a.T;
  ws.lane = lane;
  ws.c2 = a.scale_log2;
  ws.slope2 = ALIBI ? alibi_slope(a.alibi, head, a.H) * 1.4426950408889634f : 0.f;
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    ws.m_run[j] = -INFINITY;
    ws.l_run[j] = 0.f;
#pragma unroll
    for (int mb = 0; mb < HD / 32; ++mb) ws.oacc[j][mb] = f32x16{};
  }

  // ---- Q rows -> B operands (rotated in fp32, rounded to bf16). When it fits
  // in LDS, the rotary cos/sin of the workgroup's bm rows are computed once
  // (layout [pair][row], so lanes reading consecutive rows hit distinct banks)
  // and shared by the waves of all heads in the workgroup.
  {
    const bool table = a.rope && (HD / 2) * gm.bm * (int)sizeof(float2) <= STAGES * C::STAGE;
    float2* cs = reinterpret_cast<float2*>(smem);  // [HD/2][bm]
    if (table) {
      for (int e = tid; e < (HD / 2) * gm.bm; e += NT) {
        const int r = e % gm.bm, p = e / gm.bm;
        float c, sn;
        rope_cos_sin(a.pos0 + q0 + r, a.freqs.rev[p], c, sn);
        cs[e] = make_float2(c, sn);
      }
      __syncthreads();
    }
    // rotate one 16-byte chunk (4 pairs, starting at pair p0) of query row qr
    auto rotate = [&](uint4 raw, int qr, int p0) {
      uint32_t d[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float c, sn;
        if (table) {
          const float2 t = cs[(p0 + p) * gm.bm + (qr - q0)];
          c = t.x;
          sn = t.y;
        } else {
          rope_cos_sin(a.pos0 + qr, a.freqs.rev[p0 + p], c, sn);
        }
        const uint32_t x = comp(raw, p);
        const float x0 = bf16_bits_to_f32(x & 0xffffu), x1 = bf16_bits_to_f32(x >> 16);
        d[p] = pack_bf16x2(rot0(x0, x1, c, sn), rot1(x0, x1, c, sn));
      }
      return as_bf16x8(make_uint4(d[0], d[1], d[2], d[3]));
    };
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const int qr = ws.qi + 32 * j;
      const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                                        (((long)b * a.H + head) * a.T + min(qr, a.T - 1)) * HD);
      uint4 raw[HD / 16];
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) raw[s] = src[2 * s + hf];
      if (!a.rope) {
#pragma unroll
        for (int s = 0; s < HD / 16; ++s) ws.qf[j][s] = as_bf16x8(raw[s]);
      } else if (table) {
#pragma unroll
        for (int s = 0; s < HD / 16; ++s) ws.qf[j][s] = rotate(raw[s], qr, 8 * s + 4 * hf);
      } else {
#pragma unroll
        for (int s = 0; s < HD / 16; ++s) ws.qf[j][s] = rotate(raw[s], qr, 8 * s + 4 * hf);
      }
    }
    if (table) __syncthreads();  // the table area is reused by the K/V tiles
  }

  st.store(smem, tid);
  if constexpr (STAGES == 3) {
    if (nkt > 1) st.load(Kg, Vg, 1, a.T, tid);
  }
  __syncthreads();

  // Tiles [0, kt_clean) need no mask for any row of the workgroup: every key is
  // at or before the first query row (causal) and inside the sequence.
  const int kt_clean = min(nkt, CAUSAL ? min((q0 + 1) / BN, a.T / BN) : a.T / BN);
  auto step = [&](int kt, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int k0 = kt * BN;
    if constexpr (STAGES == 3) {
      // registers hold tile kt+1 (loaded one step ago): store it, then fetch kt+2
      if (kt + 1 < nkt) st.store(smem + ((kt + 1) % 3) * C::STAGE, tid);
      if (kt + 2 < nkt) st.load(Kg, Vg, kt + 2, a.T, tid);
    } else {
      if (kt + 1 < nkt) st.load(Kg, Vg, kt + 1, a.T, tid);
    }
    const unsigned char* kb = smem + (kt % STAGES) * C::STAGE;
    const bool run = wave_active && !(MASK && CAUSAL && k0 > qw0 + 32 * QB - 1);
    if (run) ws.template tile<MASK>(kb, k0);
    if constexpr (STAGES == 2) {
      if (kt + 1 < nkt) st.store(smem + ((kt + 1) & 1) * C::STAGE, tid);
    }
    __syncthreads();
  };
  int kt = 0;
  for (; kt < kt_clean; ++kt) step(kt, std::integral_constant<bool, false>{});
  for (; kt < nkt; ++kt) step(kt, std::integral_constant<bool, true>{});

  if (!wave_active) return;
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const float l_tot = ws.l_run[j] + xhalf(ws.l_run[j]);
    const int qi = ws.qi + 32 * j;
    if (qi >= a.T) continue;
    const float inv_l = 1.0f / l_tot;
    const long orow = (((long)b * a.H + head) * a.T + qi) * HD;
#pragma unroll
    for (int mb = 0; mb < HD / 32; ++mb) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * mb + 8 * g4 + 4 * hf;
        const float o0 = ws.oacc[j][mb][4 * g4 + 0] * inv_l, o1 = ws.oacc[j][mb][4 * g4 + 1] * inv_l;
        const float o2 = ws.oacc[j][mb][4 * g4 + 2] * inv_l, o3 = ws.oacc[j][mb][4 * g4 + 3] * inv_l;
        if constexpr (OUT_BF16) {
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + orow + d) =
              make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + orow + d) = make_float4(o0, o1, o2, o3);
        }
      }
    }
    if (a.lse && hf == 0) a.lse[((long)b * a.H + head) * a.T + qi] = (ws.m_run[j] + log2f(l_tot)) * 0.69314718055994531f;
  }
}

constexpr int kQB = 1;  // query blocks of 32 rows per wave in the launched kernels

GridMap make_grid(const PrefillArgs& a) {
  GridMap gm;
  gm.hpw = (a.group % 4 == 0) ? 4 : (a.group % 2 == 0 ? 2 : 1);
  gm.hchunks = a.group / gm.hpw;
  gm.bm = 32 * kQB * (NW / gm.hpw);
  gm.nqb = (a.T + gm.bm - 1) / gm.bm;
  gm.units = a.B * a.KV * gm.hchunks;
  gm.xcd_aware = (gm.units % 8) == 0;
  return gm;
}

template <int HD, bool ALIBI, bool CAUSAL>
void launch_out(const PrefillArgs& a, const GridMap& gm, dim3 grid, hipStream_t s) {
  if (a.out_bf16) {
    hipLaunchKernelGGL((prefill_mfma_kernel<HD, ALIBI, CAUSAL, true, kQB>), grid, dim3(NT), 0, s, a, gm);
  } else {
    hipLaunchKernelGGL((prefill_mfma_kernel<HD, ALIBI, CAUSAL, false, kQB>), grid, dim3(NT), 0, s, a, gm);
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
