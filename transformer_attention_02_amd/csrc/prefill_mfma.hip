// bf16 matrix-core prefill kernel for gfx950 (CDNA4).
//
// Computes the tiled online-softmax attention forward ("Building Grouped-Query
// Attention with RoPE and Flash Attention from Scratch", Step 3; recurrences of
// "Building a Transformer from Scratch", Part 3) with bf16 operands and fp32
// softmax statistics and accumulation (that page's mixed-precision roadmap item).
//
// Work decomposition
//   * A workgroup is 8 waves (two per SIMD). It owns one block of query rows
//     for up to 4 query heads that share one key/value head (grouped-query
//     packing), so every K/V tile staged in LDS serves 256 query rows.
//   * A wave owns 32 query rows of one head and computes S^T = K Q^T with
//     v_mfma_f32_32x32x16_bf16. In the 32x32 accumulator a lane holds one
//     query (column) and 16 keys (rows), so the row max and row sum are
//     in-lane reductions plus one exchange between the two half-waves.
//   * The key rows fed to the S^T contraction are permuted (bits 2 and 3 of
//     the row index swapped) so that accumulator registers 8u..8u+7 of a lane
//     hold 8 consecutive keys: the probabilities then feed O^T = V^T P^T as the
//     B operand straight from registers (rounded to bf16).
//   * The V^T P^T product of tile j is deferred to tile j+1 and issued between
//     the instructions of tile j+1's softmax: the matrix core and the vector
//     ALU of one wave then work at the same time.
//   * K/V tiles of 64 keys go global -> LDS by DMA (buffer loads that write LDS
//     directly) into a 3-stage ring: tile j+1 lands while tile j is computed
//     and V of tile j-1 is still read. Tiles are stored row-major with XOR-
//     swizzled 16-byte chunks; V^T operands are read with ds_read_b64_tr_b16
//     (the transposing LDS load of gfx950).
//   * Causal: tiles past the diagonal are never loaded; a wave skips tiles that
//     are entirely above its rows; only tiles crossing the diagonal (or the
//     ragged end of the sequence) are masked.
//   * Rotary embedding of Q is fused into the Q load (fp32 rotation, rounded to
//     bf16); K arrives already rotated (a pre-pass writes it once).
//   * Workgroups are numbered so that every workgroup touching one key/value
//     head lands on the same XCD (its L2 keeps that head's K/V), heaviest
//     causal blocks first.
#include <type_traits>

#include "mfma_tile.h"

namespace attn {

namespace {

using namespace tile;

constexpr int NW = 8;   // waves per workgroup (two per SIMD)
constexpr int kKAhead = 4;       // K operand reads issued ahead of the score MFMAs
constexpr int kValuPerMfma = 8;  // softmax instructions issued per deferred V^T MFMA
constexpr int NT = NW * 64;

struct GridMap {
  int hpw;       // heads per workgroup (1, 2 or 4)
  int hchunks;   // group / hpw
  int bm;        // query rows per head per workgroup = 32 * (NW / hpw)
  int nqb;       // query blocks
  int units;     // B * KV * hchunks
  int xcd_aware;
};

__device__ __forceinline__ float xhalf(float x) { return __shfl_xor(x, 32); }

// One wave's online-softmax state for 32 query rows (lane n holds row qi, the
// two half-waves split the keys of a tile), and the steps of one 64-key tile.
template <int HD, bool ALIBI, bool CAUSAL, bool WINDOW>
struct WaveState {
  f32x16 oacc[HD / 32];  // O^T: lane holds query n, dims 32mb + 8(r/4) + 4hf + r%4
  bf16x8 qf[HD / 16];    // Q^T B operand, k-step s: dims 16s + 8hf .. +7
  bf16x8 pprev[4];       // P^T operands (keys 16u + 8hf .. +7) whose V^T product is still due
  float m_run;           // running max (log2 units)
  float l_run;           // this half-wave's part of the running denominator
  float c2;              // log2(e) / sqrt(hd)
  float slope2;          // ALiBi slope * log2(e)
  int qi;                // this lane's query token (index in the key sequence)
  int Tk;                // keys in the sequence
  int window;            // sliding window in tokens (0: none)
  int lane;
  int vtr[HD / 32];      // byte offset in the V tile of this lane's V^T read, key row 8hf + (lane%16)/4

  // The offsets are made opaque to the optimizer: otherwise it re-derives
  // each address from a neighbouring one in long pointer chains, and the
  // compiler then can no longer tell which LDS stage a read touches and waits
  // for the DMA into another stage before it.
  __device__ __forceinline__ void init_offsets() {
    const int li = lane & 15, hf = lane >> 5;
#pragma unroll
    for (int mb = 0; mb < HD / 32; ++mb) {
      const int col = 32 * mb + 16 * ((lane >> 4) & 1) + 4 * (li & 3);
      int o = v_off<HD>(8 * hf + (li >> 2), col >> 3) + (col & 7) * 2;
#if defined(__HIP_DEVICE_COMPILE__)
      asm volatile("" : "+v"(o));
#endif
      vtr[mb] = o;
    }
  }

  // S^T = K Q^T for the 64 keys of the K tile at kb. The K rows are read in
  // permuted order (perm_row) so that register i of s[i/16] holds key
  // k0 + 32(i/16) + 16((i%16)/8) + 8hf + i%8.
  __device__ __forceinline__ void scores(LdsBytes kb, f32x16& sa, f32x16& sb) const {
    const int n = lane & 31, hf = lane >> 5;
    const int krow = perm_row(n);
    sa = f32x16{};
    sb = f32x16{};
#pragma unroll
    for (int s = 0; s < HD / 16; ++s) {
      const bf16x8 av = *reinterpret_cast<const LDS bf16x8*>(kb + k_off<HD>(krow, 2 * s + hf));
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[s], sa, 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < HD / 16; ++s) {
      const bf16x8 av = *reinterpret_cast<const LDS bf16x8*>(kb + k_off<HD>(32 + krow, 2 * s + hf));
      sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[s], sb, 0, 0, 0);
    }
    // Issue order: kKAhead operand reads go out before the first MFMA, then
    // one read per MFMA, so LDS latency hides behind kKAhead MFMAs.
    constexpr int NR = 2 * (HD / 16);
    __builtin_amdgcn_sched_group_barrier(0x100, kKAhead, 0);
#pragma unroll
    for (int i = 0; i < NR - kKAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kKAhead, 0);
  }

  // O^T += V^T P^T over four 16-key steps of the V tile at vb. V^T is read
  // with transposing loads: source lane i of a 16-lane group points at key row
  // 16u + 8hf + i/4 (+4), columns d0 + 4(i%4), and lane i then holds
  // V[those 4 keys][d0 + i].
  __device__ __forceinline__ void pv(LdsBytes vb, const bf16x8 (&p)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int mb = 0; mb < HD / 32; ++mb) {
        LdsBytes q = vb + vtr[mb] + 16 * u * HD * 2;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)q);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(q + 4 * HD * 2));
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, p[u], oacc[mb], 0, 0, 0);
      }
    }
  }

  // Online softmax of the tile whose scores are sa, sb (keys k0 .. k0+63),
  // interleaved with the V^T product of the previous tile (V tile at vprev,
  // operands pprev): the two are independent, so the vector ALU works while
  // the matrix core runs. The previous product enters O before O is rescaled
  // for this tile's max, so O and l stay at the same reference max.
  template <bool MASK>
  __device__ __forceinline__ void softmax_pv(const f32x16& sa, const f32x16& sb, int k0, LdsBytes vprev) {
    const int hf = lane >> 5;
    // Without ALiBi t keeps the raw scores (the max commutes with the positive
    // scale, which is folded into the exponent's FMA); with ALiBi t is the
    // scaled, biased score in log2 units.
    float t[32];
    const int dbase = k0 + 8 * hf - qi;  // key - query at register offset 0
    // ALiBi: register i sits at key - query = dbase + c_i with a constant c_i, so
    // the bias costs one FMA per score when causal (slope2 * dbase is formed once;
    // distances are exact in fp32) and an add plus a multiply otherwise.
    const float dbf = (float)dbase;
    const float sbase = slope2 * dbf;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float x = i < 16 ? sa[i] : sb[i - 16];
      if constexpr (ALIBI) {
        const float ci = (float)(32 * (i / 16) + 16 * ((i % 16) / 8) + (i % 8));
        const float bias = CAUSAL ? fmaf(slope2, ci, sbase) : -slope2 * fabsf(dbf + ci);
        t[i] = fmaf(x, c2, bias);
      } else {
        t[i] = x;
      }
    }
    if constexpr (MASK) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int dk = dbase + 32 * (i / 16) + 16 * ((i % 16) / 8) + (i % 8);
        const bool vis = (dk + qi < Tk) && (!CAUSAL || dk <= 0) && (!WINDOW || dk > -window);
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
    // 1), so no row's arithmetic depends on another row's scores.
    const bool move = ms > m_run + 8.0f;
    const float alpha = move ? __builtin_amdgcn_exp2f(m_run - ms) : 1.0f;
    m_run = move ? ms : m_run;
    // A masked tile can hold no visible key for a row that has seen none yet
    // (a sliding window starting inside a later tile): its weights must come
    // out as exact zeros, not as exp2(-inf - (-inf)).
    const float mref = (MASK && m_run == -INFINITY) ? 0.f : m_run;
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      t[i] = __builtin_amdgcn_exp2f(ALIBI ? t[i] - mref : fmaf(t[i], c2, -mref));
      ls[i % 4] += t[i];
    }
    l_run = fmaf(l_run, alpha, (ls[0] + ls[1]) + (ls[2] + ls[3]));
    bf16x8 pnew[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      pnew[u] = as_bf16x8(make_uint4(pack_bf16x2(t[8 * u + 0], t[8 * u + 1]), pack_bf16x2(t[8 * u + 2], t[8 * u + 3]),
                                     pack_bf16x2(t[8 * u + 4], t[8 * u + 5]), pack_bf16x2(t[8 * u + 6], t[8 * u + 7])));
    pv(vprev, pprev);
#if defined(__HIP_DEVICE_COMPILE__)
    // The probabilities are needed only after the rescale branch below; pin
    // them here so that the compiler does not sink the softmax past the branch
    // (out of reach of the interleaving).
#pragma unroll
    for (int u = 0; u < 4; ++u) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, pnew[u])));
    asm volatile("" ::"v"(l_run));
#endif
    // Issue order: the first two V^T operands, then per MFMA a slice of the
    // softmax and the next operand.
    constexpr int NM = 4 * (HD / 32);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    if (__any(move)) {
      // (a side effect keeps this a real branch: the compiler would otherwise
      // hoist the multiplies, which are an identity when no row moves)
      asm volatile("; rescale" ::: "memory");
#pragma unroll
      for (int mb = 0; mb < HD / 32; ++mb) oacc[mb] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) pprev[u] = pnew[u];
  }
};

template <int HD, bool ALIBI, bool CAUSAL, bool OUT_BF16, bool WINDOW>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_mfma_kernel(PrefillArgs a, GridMap gm) {
  using C = Cfg<HD>;
  // Three stage buffers, each its own LDS object: stage kt%3 holds tile kt
  // (K then V), stage (kt+1)%3 receives tile kt+1 by DMA, stage (kt-1)%3 still
  // holds V of tile kt-1 for its deferred V^T product. As separate objects the
  // compiler can tell that the DMA into one stage cannot alias the reads of
  // another, and does not wait for the in-flight tile before reading.
  __shared__ __attribute__((aligned(16))) unsigned char s0[C::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char s1[C::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char s2[C::STAGE];

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
  const bool wave_active = qw0 < a.Tq;

  const long kvoff = ((long)b * a.KV + kvh) * (long)a.Tk * HD;
  const uint16_t* Kg = reinterpret_cast<const uint16_t*>(a.k) + kvoff;
  const uint16_t* Vg = reinterpret_cast<const uint16_t*>(a.v) + kvoff;
  const int q_last = min(a.Tq, q0 + gm.bm) - 1;
  // Query rows are key tokens q_off + row. Key tiles [kt_begin, nkt) hold every
  // key some row of the workgroup sees: up to the last row's own token
  // (causal), from the first row's window start (sliding window).
  const int tq0 = a.q_off + q0, tq_last = a.q_off + q_last;
  const int nkt = CAUSAL ? (tq_last / BN + 1) : (a.Tk + BN - 1) / BN;
  const int kt_begin = WINDOW ? max(0, tq0 - a.window + 1) / BN : 0;

  // The first K/V tile streams into stage 0 during the Q set-up.
  Dma<HD, NW> dma;
  dma.init(wave, lane);
  dma.issue(Kg, Vg, kt_begin, a.Tk, s0, wave);
  // Stage 2 stands in for the tile before the first one: its V part is zeroed
  // and the pending probabilities start at zero, so the first tile's deferred
  // product adds exact zeros.
  for (int e = tid; e < C::V_BYTES / 16; e += NT) reinterpret_cast<uint4*>(s2 + C::K_BYTES)[e] = make_uint4(0, 0, 0, 0);

  WaveState<HD, ALIBI, CAUSAL, WINDOW> ws;
  ws.qi = a.q_off + qw0 + n;
  ws.Tk = a.Tk;
  ws.window = a.window;
  ws.lane = lane;
  ws.init_offsets();
  ws.c2 = a.scale_log2;
  ws.slope2 = ALIBI ? alibi_slope(a.alibi, head, a.H) * 1.4426950408889634f : 0.f;
  ws.m_run = -INFINITY;
  ws.l_run = 0.f;
#pragma unroll
  for (int mb = 0; mb < HD / 32; ++mb) ws.oacc[mb] = f32x16{};
#pragma unroll
  for (int u = 0; u < 4; ++u) ws.pprev[u] = as_bf16x8(make_uint4(0, 0, 0, 0));

  // ---- Q rows -> B operands (rotated in fp32, rounded to bf16). When it fits
  // in stage 1, the rotary cos/sin of the workgroup's bm rows are computed once
  // (layout [pair][row], so lanes reading consecutive rows hit distinct banks)
  // and shared by the waves of all heads in the workgroup.
  {
    const bool table = a.rope && (HD / 2) * gm.bm * (int)sizeof(float2) <= C::STAGE;
    float2* cs = reinterpret_cast<float2*>(s1);  // [HD/2][bm]
    if (table) {
      for (int e = tid; e < (HD / 2) * gm.bm; e += NT) {
        const int r = e % gm.bm, p = e / gm.bm;
        float c, sn;
        rope_cos_sin(a.pos0 + tq0 + r, a.freqs.rev[p], c, sn);
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
          rope_cos_sin(a.pos0 + a.q_off + qr, a.freqs.rev[p0 + p], c, sn);
        }
        const uint32_t x = comp(raw, p);
        const float x0 = bf16_bits_to_f32(x & 0xffffu), x1 = bf16_bits_to_f32(x >> 16);
        d[p] = pack_bf16x2(rot0(x0, x1, c, sn), rot1(x0, x1, c, sn));
      }
      return as_bf16x8(make_uint4(d[0], d[1], d[2], d[3]));
    };
    const int qr = qw0 + n;  // query row
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                                      (((long)b * a.H + head) * a.Tq + min(qr, a.Tq - 1)) * HD);
    uint4 raw[HD / 16];
#pragma unroll
    for (int s = 0; s < HD / 16; ++s) raw[s] = src[2 * s + hf];
    if (!a.rope) {
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) ws.qf[s] = as_bf16x8(raw[s]);
    } else {
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) ws.qf[s] = rotate(raw[s], qr, 8 * s + 4 * hf);
    }
  }
  // Tile 0 has landed, stage 2 is zeroed and no wave still reads the table (stage 1).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Tiles [kc_lo, kc_hi) need no mask for any row of the workgroup: every key
  // is at or before the first row's token (causal), inside the last row's
  // window and inside the sequence.
  const int kc_lo = WINDOW ? max(kt_begin, (max(0, tq_last - a.window + 1) + BN - 1) / BN) : kt_begin;
  const int kc_hi = min(nkt, CAUSAL ? min((tq0 + 1) / BN, a.Tk / BN) : a.Tk / BN);
  // Per tile: start the DMA of tile kt+1, the scores of tile kt, then its
  // softmax under the deferred V^T product of tile kt-1; the wait + barrier at
  // the end publishes tile kt+1 and retires stage kt-1.
  // pprev owes its V^T product. Without a window every active wave runs the
  // first tile, so this starts true (the zero operands of "tile -1" are
  // harmless); with a window a wave may skip the first tiles and starts false.
  bool pending = !WINDOW;
  auto step = [&](int kt, auto mask_tag, auto phase_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int P = decltype(phase_tag)::value;
    unsigned char* cur = P == 0 ? s0 : (P == 1 ? s1 : s2);
    unsigned char* prv = P == 0 ? s2 : (P == 1 ? s0 : s1);
    unsigned char* nxt = P == 0 ? s1 : (P == 1 ? s2 : s0);
    const int k0 = kt * BN;
    if (kt + 1 < nkt) dma.issue(Kg, Vg, kt + 1, a.Tk, nxt, wave);
    // in a masked tile a wave may be past its last visible key (causal) or
    // before its first one (sliding window)
    const int tw0 = a.q_off + qw0;
    const bool run = wave_active && !(MASK && ((CAUSAL && k0 > tw0 + 31) ||
                                               (WINDOW && k0 + BN - 1 < tw0 - a.window + 1)));
    if (run) {
      f32x16 sa, sb;
      ws.scores((LdsBytes)cur, sa, sb);
      // A wave in its softmax + deferred-product phase gets issue priority
      // over a wave computing scores (measured: fewer cycles per tile).
      __builtin_amdgcn_s_setprio(1);
      ws.template softmax_pv<MASK>(sa, sb, k0, (LdsBytes)(prv + C::K_BYTES));
      __builtin_amdgcn_s_setprio(0);
      if constexpr (MASK && WINDOW) pending = true;
    } else if (MASK && pending) {
      // past the wave's last visible key: settle the owed product (the wave
      // does not run again)
      ws.pv((LdsBytes)(prv + C::K_BYTES), ws.pprev);
      pending = false;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  using F = std::integral_constant<bool, false>;
  using M = std::integral_constant<bool, true>;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  // Tile kt uses ring stage (kt - kt_begin) % 3, and every loop below starts a
  // round of the ring at stage 0, so each step names its stages statically.
  // Masked rounds run the masked step, which is also correct for clean tiles.
  int kt = kt_begin;
  auto masked_rounds = [&](int end) __attribute__((always_inline)) {
    while (kt < end) {
      step(kt, M{}, P0{});
      if (++kt >= end) break;
      step(kt, M{}, P1{});
      if (++kt >= end) break;
      step(kt, M{}, P2{});
      ++kt;
    }
  };
  if constexpr (WINDOW) {
    // tiles at the window's start, up to the first round boundary at or after
    // the first clean tile
    masked_rounds(min(nkt, kt_begin + (kc_lo - kt_begin + 2) / 3 * 3));
  }
  if constexpr (WINDOW) {
    if (kt + 3 <= kc_hi) pending = true;  // every active wave runs a clean tile
  }
  for (; kt + 3 <= kc_hi; kt += 3) {
    step(kt, F{}, P0{});
    step(kt + 1, F{}, P1{});
    step(kt + 2, F{}, P2{});
  }
  masked_rounds(nkt);
  if (!wave_active) return;
  // the last tile's V^T product (no DMA is in flight any more)
  if (pending) {
    const int p = (nkt - 1 - kt_begin) % 3;
    ws.pv((LdsBytes)((p == 0 ? s0 : (p == 1 ? s1 : s2)) + C::K_BYTES), ws.pprev);
  }

  const float l_tot = ws.l_run + xhalf(ws.l_run);
  const int qi = qw0 + n;  // query row
  if (qi >= a.Tq) return;
  const float inv_l = 1.0f / l_tot;
  const long orow = (((long)b * a.H + head) * a.Tq + qi) * HD;
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
  if (a.lse && hf == 0) a.lse[((long)b * a.H + head) * a.Tq + qi] = (ws.m_run + log2f(l_tot)) * 0.69314718055994531f;
}

GridMap make_grid(const PrefillArgs& a) {
  GridMap gm;
  gm.hpw = (a.group % 4 == 0) ? 4 : (a.group % 2 == 0 ? 2 : 1);
  gm.hchunks = a.group / gm.hpw;
  gm.bm = 32 * (NW / gm.hpw);
  gm.nqb = (a.Tq + gm.bm - 1) / gm.bm;
  gm.units = a.B * a.KV * gm.hchunks;
  gm.xcd_aware = (gm.units % 8) == 0;
  return gm;
}

template <int HD, bool ALIBI, bool CAUSAL, bool WINDOW>
void launch_out(const PrefillArgs& a, const GridMap& gm, dim3 grid, hipStream_t s) {
  if (a.out_bf16) {
    hipLaunchKernelGGL((prefill_mfma_kernel<HD, ALIBI, CAUSAL, true, WINDOW>), grid, dim3(NT), 0, s, a, gm);
  } else {
    hipLaunchKernelGGL((prefill_mfma_kernel<HD, ALIBI, CAUSAL, false, WINDOW>), grid, dim3(NT), 0, s, a, gm);
  }
}

// The sliding window is a separate instance (causal only), so the plain
// kernels carry none of its masking or tile-skipping code.
template <int HD>
void launch_hd(const PrefillArgs& a, const GridMap& gm, dim3 grid, hipStream_t s) {
  if (a.alibi) {
    if (a.window > 0) launch_out<HD, true, true, true>(a, gm, grid, s);
    else if (a.causal) launch_out<HD, true, true, false>(a, gm, grid, s);
    else launch_out<HD, true, false, false>(a, gm, grid, s);
  } else {
    if (a.window > 0) launch_out<HD, false, true, true>(a, gm, grid, s);
    else if (a.causal) launch_out<HD, false, true, false>(a, gm, grid, s);
    else launch_out<HD, false, false, false>(a, gm, grid, s);
  }
}

}  // namespace

bool prefill_mfma_supported(const PrefillArgs& a, int bf16) {
  if (!bf16 || (a.hd != 64 && a.hd != 128)) return false;
  if ((long)a.Tk * a.hd * 2 >= (1L << 31)) return false;  // buffer descriptors hold 32-bit sizes
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
