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
constexpr int kKAhead = 8;  // K operand reads in flight ahead of the score MFMAs
constexpr int NT = NW * 64;

template <int HD>
struct Cfg {
  static constexpr int KCH = HD / 8;               // 16-byte chunks per key row
  static constexpr int K_BYTES = BN * HD * 2;      // K tile, row-major [key][hd], XOR-swizzled chunks
  static constexpr int V_BYTES = BN * HD * 2;      // V tile, row-major [key][hd], XOR-swizzled chunks
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int DMA = K_BYTES / 1024;       // 1 KiB LDS-DMA wave instructions per tensor per tile
};

struct GridMap {
  int hpw;       // heads per workgroup (1, 2 or 4)
  int hchunks;   // group / hpw
  int bm;        // query rows per head per workgroup = 32 * QB * (4 / hpw)
  int nqb;       // query blocks
  int units;     // B * KV * hchunks
  int xcd_aware;
};

// XOR swizzles of the 16-byte chunk index. Rows are unpadded (so one LDS-DMA
// wave instruction fills 1 KiB of whole rows) and the swizzles keep every MFMA
// operand read free of bank conflicts (measured: SQ_LDS_BANK_CONFLICT = 0):
//  * K: the 16 lanes of a ds_read_b128 read one logical chunk of 16 different
//    rows; XOR with the row's low bits sends them to 16 different chunk slots;
//  * V: a transposing load reads rows r..r+3 x 32 bytes per 16-lane group (64
//    bytes per 32 lanes); XOR with (r & 3) << 2 moves each row to its own
//    64-byte bank range.
template <int HD>
__host__ __device__ constexpr int k_swz(int r) {
  return HD == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int HD>
__host__ __device__ constexpr int v_swz(int r) {
  return HD == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}
// Byte offset of logical 16-byte chunk `c` of key row `r` in the K / V tile.
template <int HD>
__host__ __device__ constexpr int k_off(int r, int c) { return r * HD * 2 + ((c ^ k_swz<HD>(r)) << 4); }
template <int HD>
__host__ __device__ constexpr int v_off(int r, int c) { return r * HD * 2 + ((c ^ v_swz<HD>(r)) << 4); }

// The V swizzle depends on the row only through bits that a step of 4 rows
// keeps, so each lane's transposing-load addresses for the rows r + 4e + 16u
// are its row-r address plus a constant (an instruction offset).
template <int HD>
constexpr bool v_rows_affine() {
  for (int r0 = 0; r0 < 12; ++r0)
    for (int d = 0; d < 64 - 12; d += 4)
      for (int c = 0; c < HD / 8; ++c)
        if (v_off<HD>(r0 + d, c) != v_off<HD>(r0, c) + d * HD * 2) return false;
  return true;
}
static_assert(v_rows_affine<64>() && v_rows_affine<128>(), "V swizzle must be invariant under 4-row steps");

// Swap bits 2 and 3 of a row index in [0, 32).
__device__ __forceinline__ int perm_row(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Component i (a compile-time constant after unrolling) of a uint4, without taking its address.
__device__ __forceinline__ uint32_t comp(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ float xhalf(float x) { return __shfl_xor(x, 32); }

#define LDS __attribute__((address_space(3)))
typedef const LDS unsigned char* LdsBytes;  // operand reads address LDS directly

// Direct global -> LDS staging of one K/V tile (no registers in between). Wave
// w issues wave instructions q = w*DMA/4 .. of 1 KiB each per tensor; lane l of
// instruction q fills LDS bytes 1024q + 16l, i.e. key row r = (1024q + 16l) /
// (2hd) at physical chunk pc, so it fetches the logical chunk pc ^ swz(r) of
// that row. The buffer descriptor starts at the tile and ends at the slab end:
// rows at or past T are written as zeros.
template <int HD>
struct Dma {
  using C = Cfg<HD>;
  static constexpr int PER_WAVE = C::DMA / NW;
  int koff[PER_WAVE];  // per-lane source byte offsets within the tile
  int voff[PER_WAVE];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int p = 1024 * (wave * PER_WAVE + i) + 16 * lane;
      const int r = p / (HD * 2), pc = (p % (HD * 2)) / 16;
      koff[i] = (r * HD + (pc ^ k_swz<HD>(r)) * 8) * 2;
      voff[i] = (r * HD + (pc ^ v_swz<HD>(r)) * 8) * 2;
    }
  }

  __device__ __forceinline__ void issue(const uint16_t* Kg, const uint16_t* Vg, int kt, int T, unsigned char* stage,
                                        int wave) const {
    const int bytes = (T - kt * BN) * HD * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg + (long)kt * BN * HD, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg + (long)kt * BN * HD, bytes);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = wave * PER_WAVE + i;
#if defined(__HIP_DEVICE_COMPILE__)  // (the host pass drops the kernel stubs of later instantiations otherwise)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LDS void*)(stage + 1024 * q), 16, koff[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LDS void*)(stage + C::K_BYTES + 1024 * q), 16, voff[i], 0, 0, 0);
#endif
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
  int vtr[HD / 32];          // byte offset (from the K tile start) of this lane's V^T read, key row 8hf + (lane%16)/4

  // The offsets are made opaque to the optimizer: otherwise it re-derives
  // each address from a neighbouring one in long pointer chains, and the
  // compiler then can no longer tell which LDS stage a read touches and waits
  // for the DMA into the other stage before it.
  __device__ __forceinline__ void init_offsets() {
    using C = Cfg<HD>;
    const int li = lane & 15, hf = lane >> 5;
#pragma unroll
    for (int mb = 0; mb < HD / 32; ++mb) {
      const int col = 32 * mb + 16 * ((lane >> 4) & 1) + 4 * (li & 3);
      int o = C::K_BYTES + v_off<HD>(8 * hf + (li >> 2), col >> 3) + (col & 7) * 2;
#if defined(__HIP_DEVICE_COMPILE__)
      asm volatile("" : "+v"(o));
#endif
      vtr[mb] = o;
    }
  }

  template <bool MASK>
  __device__ __forceinline__ void tile(LdsBytes kb, int k0) {
    using C = Cfg<HD>;
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
        const bf16x8 av = *reinterpret_cast<const LDS bf16x8*>(kb + k_off<HD>(32 * kb2 + krow, 2 * s + hf));
#pragma unroll
        for (int j = 0; j < QB; ++j)
          sacc[j][kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[j][s], sacc[j][kb2], 0, 0, 0);
      }
    }
    // Issue order of the score products: the first kKAhead operand reads go
    // out before any MFMA, then one read per MFMA, so LDS latency hides behind
    // kKAhead MFMAs instead of one.
    {
      constexpr int NR = 2 * (HD / 16), NM = NR * QB;
      __builtin_amdgcn_sched_group_barrier(0x100, kKAhead, 0);
#pragma unroll
      for (int i = 0; i < NR - kKAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NM - QB * (NR - kKAhead), 0);
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
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int mb = 0; mb < HD / 32; ++mb) {
        LdsBytes p = kb + vtr[mb] + 16 * u * HD * 2;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)p);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(p + 4 * HD * 2));
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int j = 0; j < QB; ++j)
          if (live[j]) oacc[j][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[j][u], oacc[j][mb], 0, 0, 0);
      }
    }
  }
};

// QB = query blocks of 32 rows per wave: QB = 1 runs two waves per SIMD, QB = 2
// one (its state needs ~400 VGPRs).
template <int QB>
struct Sched {
  static constexpr int WAVES_PER_EU = QB == 2 ? 1 : 2;
};

template <int HD, bool ALIBI, bool CAUSAL, bool OUT_BF16, int QB>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(Sched<QB>::WAVES_PER_EU, Sched<QB>::WAVES_PER_EU)))
void prefill_mfma_kernel(PrefillArgs a, GridMap gm) {
  using C = Cfg<HD>;
  // Two stage buffers as separate LDS objects: the compiler then knows that the
  // DMA filling one stage cannot alias the reads of the other, and does not
  // wait for the in-flight tile before reading the current one.
  __shared__ __attribute__((aligned(16))) unsigned char s0[C::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char s1[C::STAGE];

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

  // The first K/V tile streams into stage 0 during the Q set-up.
  Dma<HD> dma;
  dma.init(wave, lane);
  dma.issue(Kg, Vg, 0, a.T, s0, wave);

  WaveState<HD, ALIBI, CAUSAL, QB> ws;
  ws.qi = qw0 + n;
  ws.T = a.T;
  ws.lane = lane;
  ws.init_offsets();
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
  // in the stage-1 area, the rotary cos/sin of the workgroup's bm rows are
  // computed once (layout [pair][row], so lanes reading consecutive rows hit
  // distinct banks) and shared by the waves of all heads in the workgroup.
  {
    const bool table = a.rope && (HD / 2) * gm.bm * (int)sizeof(float2) <= C::STAGE;
    float2* cs = reinterpret_cast<float2*>(s1);  // [HD/2][bm]
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
  }
  // Tile 0 has landed and no wave still reads the table area (stage 1).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Tiles [0, kt_clean) need no mask for any row of the workgroup: every key is
  // at or before the first query row (causal) and inside the sequence.
  const int kt_clean = min(nkt, CAUSAL ? min((q0 + 1) / BN, a.T / BN) : a.T / BN);
  // Double buffer: tile kt+1 streams into the other stage while tile kt is
  // computed; the wait + barrier at the end publishes it and retires stage kt.
  // The stage parity is a compile-time constant of each step.
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  auto step = [&](int kt, auto mask_tag, auto par_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int P = decltype(par_tag)::value;
    unsigned char* cur = P ? s1 : s0;
    unsigned char* nxt = P ? s0 : s1;
    const int k0 = kt * BN;
    if (kt + 1 < nkt) dma.issue(Kg, Vg, kt + 1, a.T, nxt, wave);
    const bool run = wave_active && !(MASK && CAUSAL && k0 > qw0 + 32 * QB - 1);
    if (run) ws.template tile<MASK>((LdsBytes)cur, k0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  int kt = 0;
  auto phase = [&](int end, auto mask_tag) __attribute__((always_inline)) {
    if (kt & 1) {
      while (kt < end) {
        step(kt++, mask_tag, Odd{});
        if (kt >= end) break;
        step(kt++, mask_tag, Even{});
      }
    } else {
      while (kt < end) {
        step(kt++, mask_tag, Even{});
        if (kt >= end) break;
        step(kt++, mask_tag, Odd{});
      }
    }
  };
  phase(kt_clean, std::integral_constant<bool, false>{});
  phase(nkt, std::integral_constant<bool, true>{});

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
