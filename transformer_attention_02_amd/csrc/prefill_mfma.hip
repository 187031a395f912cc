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
//     packing), so every K/V tile staged in LDS serves 256 query rows. A grid
//     that would not give every compute unit a workgroup runs 4-wave
//     workgroups instead (half the rows each, 80 KiB of LDS, two per compute
//     unit): twice as many workgroups share out the same work. When even
//     that grid leaves compute units idle (head size 64), the 4 waves of a
//     workgroup take the same 32 rows of one head and split their key tiles
//     four ways instead, merging the four partial states at the end.
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
//     causal blocks first; an XCD works through its heads a few at a time, as
//     many as keep their K/V within its 4 MiB L2.
#include <type_traits>

#include "mfma_tile.h"

namespace attn {

namespace {

using namespace tile;

constexpr int kKAhead = 4;       // K operand reads issued ahead of the score MFMAs
constexpr int kValuPerMfma = 8;  // softmax instructions issued per deferred V^T MFMA

struct GridMap {
  int hpw;       // heads per workgroup (1, 2 or 4)
  int hchunks;   // group / hpw
  int bm;        // query rows per head per workgroup = 32 * (waves / hpw)
  int nqb;       // query blocks
  int units;     // B * KV * hchunks
  int xcd_aware;
  int ugroup;    // units an XCD works on at a time
};

__device__ __forceinline__ float xhalf(float x) { return __shfl_xor(x, 32); }

// One wave's online-softmax state for 32 query rows (lane n holds row qi, the
// two half-waves split the keys of a tile), and the steps of one 64-key tile.
template <int HD, bool ALIBI, bool CAUSAL, bool WINDOW>
struct WaveState {
  f32x16 oacc[HD / 32];  // O^T: lane holds query n, dims 32mb + 8(r/4) + 4hf + r%4
  bf16x8 qf[HD / 16];    // Q^T B operand, k-step s: dims 16s + 8hf .. +7
  bf16x8 pprev[4];       // P^T operands (keys 16u + 8hf .. +7) whose V^T product is still due
  bf16x8 palt[4];        // the other set of the six-step clean loop (see softmax_pv)
  float m_run;           // running max (log2 units)
  float l_run;           // this half-wave's part of the running denominator
  float c2;              // log2(e) / sqrt(hd)
  float slope2;          // ALiBi slope * log2(e)
  // causal ALiBi without a window takes the key-offset part of its bias from
  // the matrix core (see init_alibi_mfma)
  static constexpr bool MB = ALIBI && CAUSAL && !WINDOW;
  bf16x8 kbias[2];       // MB: A operand of the bias k-step for the two 32-key halves
  bf16x8 qbias;          // MB: its B operand (slope2 / c2 as three bf16 parts)
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
    if constexpr (MB) {
      // the key-offset part of the causal ALiBi bias, on the matrix core
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kbias[0], qbias, sa, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kbias[1], qbias, sb, 0, 0, 0);
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
    __builtin_amdgcn_sched_group_barrier(0x008, kKAhead + (MB ? 2 : 0), 0);
  }

  // Causal ALiBi's bias is slope2 * (key - query). The part that varies inside
  // a tile, slope2 * (key - k0), comes from one more k-step of the S^T MFMAs:
  // the A-operand row of this lane is key 32 * blk + perm_row(lane % 32) of the
  // tile, and the first half-wave's k-values 0..2 hold that offset c (exact in
  // bf16) against B = slope2 / c2 = slope * sqrt(hd) split into three bf16
  // parts (each the bf16 of what the previous ones leave), so the products are
  // exact and their fp32 sum gives c * slope * sqrt(hd) to ~2^-24 relative.
  // The rest, slope2 * (k0 - qi), is one value per lane, added once.
  __device__ __forceinline__ void init_alibi_mfma() {
    const int n = lane & 31, hf = lane >> 5;
    const float sl = slope2 / c2;
    const __bf16 b0 = (__bf16)sl;
    const __bf16 b1 = (__bf16)(sl - (float)b0);
    const __bf16 b2 = (__bf16)(sl - (float)b0 - (float)b1);
    const __bf16 z = (__bf16)0.0f;
    qbias = hf == 0 ? bf16x8{b0, b1, b2, z, z, z, z, z} : bf16x8{z, z, z, z, z, z, z, z};
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const __bf16 c = (__bf16)(float)(32 * blk + perm_row(n));
      kbias[blk] = hf == 0 ? bf16x8{c, c, c, z, z, z, z, z} : bf16x8{z, z, z, z, z, z, z, z};
    }
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
  // SET selects the probability registers: 0 reads and rewrites pprev (a
  // copy at the end); in the six-step clean loop, 1 reads pprev and writes
  // palt, 2 reads palt and writes pprev, so no copy is needed and pprev holds
  // the due operands again after every six steps.
  // (full: every key of the tile is visible to every row of the wave, so a
  // masked step skips the mask; rounds of masked steps cover such tiles too)
  template <bool MASK, int SET = 0>
  __device__ __forceinline__ void softmax_pv(const f32x16& sa, const f32x16& sb, int k0, LdsBytes vprev,
                                             bool full = false) {
    bf16x8(&pin)[4] = SET == 2 ? palt : pprev;
    bf16x8(&pout)[4] = SET == 1 ? palt : pprev;
    const int hf = lane >> 5;
    // t keeps the raw scores (the max commutes with the positive scale, which
    // is folded into the exponent's FMA), except for ALiBi with a window or
    // without causality, where t is the scaled, biased score in log2 units.
    float t[32];
    const int dbase = k0 + 8 * hf - qi;  // key - query at register offset 0
    // Register i sits at key - query = dbase + c_i with a constant c_i
    // (distances are exact in fp32): with a window the causal bias costs one
    // FMA per score, without causality an add plus a multiply.
    const float dbf = (float)dbase;
    // MB: the scores arrive with slope2 / c2 * (key - k0) added; what is left
    // of the bias, slope2 * (k0 - qi), is common to the lane's row. Otherwise
    // ALiBi is applied here and t holds scaled scores in log2 units.
    const float sbase = slope2 * (float)(MB ? k0 - qi : dbase);
    constexpr bool SCALED = ALIBI && !MB;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float x = i < 16 ? sa[i] : sb[i - 16];
      if constexpr (SCALED) {
        const float ci = (float)(32 * (i / 16) + 16 * ((i % 16) / 8) + (i % 8));
        const float bias = CAUSAL ? fmaf(slope2, ci, sbase) : -slope2 * fabsf(dbf + ci);
        t[i] = fmaf(x, c2, bias);
      } else {
        t[i] = x;
      }
    }
    if (MASK && !full) {
      // register i holds key k0 + 8hf + c_i (c_i a constant): it is visible when
      // lo <= c_i <= hi, the per-lane limits folding the causal bound (key <= qi),
      // the sequence end (key < Tk) and the window start (key > qi - window)
      const int hi = min(CAUSAL ? -dbase : 0x7fffffff, Tk - 1 - k0 - 8 * hf);
      const int lo = WINDOW ? 1 - window - dbase : 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int ci = 32 * (i / 16) + 16 * ((i % 16) / 8) + (i % 8);
        const bool vis = WINDOW ? (ci <= hi && ci >= lo) : ci <= hi;
        t[i] = vis ? t[i] : -INFINITY;
      }
    }
    float mx = t[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mx = fmaxf(mx, t[i]);
    mx = fmaxf(mx, xhalf(mx));
    // tile max in log2 units
    const float ms = SCALED ? mx : (MB ? fmaf(mx, c2, sbase) : mx * c2);
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
    const float woff = MB ? sbase - mref : -mref;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      t[i] = __builtin_amdgcn_exp2f(SCALED ? t[i] - mref : fmaf(t[i], c2, woff));
      ls[i % 4] += t[i];
    }
    l_run = fmaf(l_run, alpha, (ls[0] + ls[1]) + (ls[2] + ls[3]));
    bf16x8 pnew[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      pnew[u] = as_bf16x8(make_uint4(pack_bf16x2(t[8 * u + 0], t[8 * u + 1]), pack_bf16x2(t[8 * u + 2], t[8 * u + 3]),
                                     pack_bf16x2(t[8 * u + 4], t[8 * u + 5]), pack_bf16x2(t[8 * u + 6], t[8 * u + 7])));
    pv(vprev, pin);
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
    for (int u = 0; u < 4; ++u) pout[u] = pnew[u];
  }
};

// LDS buffer I of one kernel instance: with 8 waves, stage I of K then V;
// with 4 waves, K buffer I (I = 0, 1) or V buffer I - 2 (I = 2, 3, 4). With
// wave-split workgroups (WS) every wave owns such a set of five.
template <int HD, int NW, bool ALIBI, bool CAUSAL, bool OUT_BF16, bool WINDOW, bool WS, int I>
__device__ __forceinline__ unsigned char* lds_buf() {
  __shared__ __attribute__((aligned(16))) unsigned char b[(NW == 8 ? Cfg<HD>::STAGE : Cfg<HD>::K_BYTES) * (WS ? NW : 1)];
  return b;
}

// WS (wave-split workgroups, for grids far too small to fill the chip): the
// 4 waves of a workgroup own the same 32 query rows of one head and split the
// block's key tiles four ways, each wave walking its share through its own
// LDS ring with no workgroup barrier per step (one wave per SIMD, so none
// waits on another's issue). Four times as many workgroups then spread over
// idle compute units, and the longest walk is a quarter as long. The four
// partial online-softmax states (running max, denominator, unnormalised O)
// are merged through LDS at the end, the way the block recurrence of the
// pages' tiled pass merges key blocks.
template <int HD, int NW, bool ALIBI, bool CAUSAL, bool OUT_BF16, bool WINDOW, bool WS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_mfma_kernel(PrefillArgs a, GridMap gm) {
  using C = Cfg<HD>;
  constexpr int NT = NW * 64;
  static_assert(!WS || NW == 4, "wave-split workgroups have 4 waves");
  // Each buffer is its own LDS object, so the compiler can tell that the DMA
  // into one cannot alias the reads of another, and does not wait for the
  // in-flight tile before reading.
  //  * 8 waves: three stages of K then V; stage j%3 holds walk tile j, stage
  //    (j+1)%3 receives tile j+1 by DMA, stage (j-1)%3 still holds V of tile
  //    j-1 for its deferred V^T product.
  //  * 4 waves: K of tile j in kb[j%2] (read in step j), V in vb[j%3] (read in
  //    step j+1); 80 KiB in all, so two workgroups share a compute unit.
  static_assert(NW == 8 || NW == 4, "8- or 4-wave workgroups");
  static_assert(C::K_BYTES == C::V_BYTES, "K and V buffers are interchangeable");
  const int tid = threadIdx.x;
  // (with WS the wave index picks each wave's tile range, hence every DMA's
  // buffer descriptor, which must be uniform: as a per-lane value the compiler
  // wraps each DMA in a loop over the lanes' values. Elsewhere it stays a
  // vector value: as a scalar one the 4-wave hd-128 instances spill registers.)
  const int wave = WS ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
#if defined(__HIP_DEVICE_COMPILE__)
  // The scalar kernel arguments the set-up needs are requested together, so
  // their memory latency is paid once rather than once per dependent use.
  asm volatile("" ::"s"(gm.units), "s"(gm.nqb), "s"(gm.ugroup), "s"(gm.xcd_aware), "s"(gm.hchunks), "s"(gm.hpw),
               "s"(gm.bm), "s"(a.KV), "s"(a.group), "s"(a.Tq), "s"(a.Tk), "s"(a.H), "s"(a.q_off), "s"(a.k),
               "s"(a.v), "s"(a.q), "s"(a.rope), "s"(a.pos0));
#endif
// buffer I of this wave (WS) or of the workgroup; LBW(W, I): buffer I of wave W
#define LBW(W, I) (lds_buf<HD, NW, ALIBI, CAUSAL, OUT_BF16, WINDOW, WS, (I)>() + (WS ? (W) * C::K_BYTES : 0))
#define LB(I) LBW(wave, I)
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;

  // ---- workgroup -> (unit = (b, kv head, head chunk), query block), heavy blocks first
  const int w = blockIdx.x;
  int unit, qrank;
  if (gm.xcd_aware) {
    // Consecutive workgroups go round-robin to the 8 XCDs. XCD x owns units
    // [x*upx, (x+1)*upx) and works through them in groups of gm.ugroup units
    // whose K/V fit its L2, interleaving a group's units, heaviest query
    // blocks first. (Working through one unit at a time measured slower: all
    // of an XCD's workgroups then hit the same K/V lines at once.)
    const int upx = gm.units >> 3;
    const int j = w >> 3;
    const int per_group = gm.ugroup * gm.nqb;
    const int g = j / per_group, r = j % per_group;
    const int gsz = min(gm.ugroup, upx - g * gm.ugroup);
    unit = (w & 7) * upx + g * gm.ugroup + r % gsz;
    qrank = r / gsz;
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
  const int qw0 = WS ? q0 : q0 + 32 * (wave / gm.hpw);
  const bool wave_active = qw0 < a.Tq;

  const long kvoff = ((long)b * a.KV + kvh) * (long)a.Tk * HD;
  const uint16_t* Kg = reinterpret_cast<const uint16_t*>(a.k) + kvoff;
  const uint16_t* Vg = reinterpret_cast<const uint16_t*>(a.v) + kvoff;
  const int q_last = min(a.Tq, q0 + gm.bm) - 1;
  // Query rows are key tokens q_off + row. Key tiles [kt_begin, nkt) hold every
  // key some row of the workgroup sees: up to the last row's own token
  // (causal), from the first row's window start (sliding window).
  const int tq0 = a.q_off + q0, tq_last = a.q_off + q_last;
  const int nkt_wg = CAUSAL ? (tq_last / BN + 1) : (a.Tk + BN - 1) / BN;
  const int kt_begin_wg = WINDOW ? max(0, tq0 - a.window + 1) / BN : 0;
  // This wave's tiles [kt_begin, nkt): the workgroup's, or with WS the w-th
  // of four consecutive shares (the first ones one tile longer; possibly none)
  int kt_begin = kt_begin_wg, nkt = nkt_wg;
  if constexpr (WS) {
    const int tot = nkt_wg - kt_begin_wg, q4 = tot / 4, r4 = tot % 4;
    kt_begin = kt_begin_wg + wave * q4 + min(wave, r4);
    nkt = kt_begin + q4 + (wave < r4 ? 1 : 0);
  }

  // Causal ALiBi walks the key tiles from the last one down: each row meets
  // its largest bias (the keys nearest its token) first, so its running max
  // is set at once instead of rising tile by tile (which forced a rescale of
  // O on most steps). Other variants walk upwards; the online softmax gives
  // the same result in any order, up to rounding.
  constexpr bool REV = ALIBI && CAUSAL && !WINDOW;
  // K and V of walk tile j: where they sit (P = j % 6)
  auto kbuf = [&](int P) __attribute__((always_inline)) {
    return NW == 8 ? (P % 3 == 0 ? LB(0) : (P % 3 == 1 ? LB(1) : LB(2))) : (P % 2 == 0 ? LB(0) : LB(1));
  };
  auto vbuf = [&](int P) __attribute__((always_inline)) {
    return NW == 8 ? (P % 3 == 0 ? LB(0) : (P % 3 == 1 ? LB(1) : LB(2))) + C::K_BYTES
                   : (P % 3 == 0 ? LB(2) : (P % 3 == 1 ? LB(3) : LB(4)));
  };
  // The first K/V tile streams in during the Q set-up.
  // (with WS each wave moves whole tiles into its own ring)
  constexpr int DW = WS ? 1 : NW;
  const int dwave = WS ? 0 : wave;
  Dma<HD, DW> dma;
  dma.init(dwave, lane);
  if (!WS || nkt > kt_begin) dma.issue(Kg, Vg, REV ? nkt - 1 : kt_begin, a.Tk, kbuf(0), vbuf(0), dwave);
  // V of the tile before the first one (buffer 2) is zeroed and the pending
  // probabilities start at zero, so the first tile's deferred product adds
  // exact zeros.
  for (int e = WS ? lane : tid; e < C::V_BYTES / 16; e += WS ? 64 : NT)
    reinterpret_cast<uint4*>(vbuf(2))[e] = make_uint4(0, 0, 0, 0);

  WaveState<HD, ALIBI, CAUSAL, WINDOW> ws;
  ws.qi = a.q_off + qw0 + n;
  ws.Tk = a.Tk;
  ws.window = a.window;
  ws.lane = lane;
  ws.init_offsets();
  ws.c2 = a.scale_log2;
  ws.slope2 = ALIBI ? alibi_slope(a.alibi, head, a.H) * 1.4426950408889634f : 0.f;
  if constexpr (ALIBI && CAUSAL && !WINDOW) ws.init_alibi_mfma();
  ws.m_run = -INFINITY;
  ws.l_run = 0.f;
#pragma unroll
  for (int mb = 0; mb < HD / 32; ++mb) ws.oacc[mb] = f32x16{};
#pragma unroll
  for (int u = 0; u < 4; ++u) ws.pprev[u] = as_bf16x8(make_uint4(0, 0, 0, 0));

  // ---- Q rows -> B operands (rotated in fp32, rounded to bf16). When it fits
  // in the K buffer of tile 1, the rotary cos/sin of the workgroup's bm rows
  // are computed once (layout [pair][row], so lanes reading consecutive rows
  // hit distinct banks) and shared by the waves of all heads in the workgroup.
  {
    const int qr = qw0 + n;  // query row
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                                      (((long)b * a.H + head) * a.Tq + min(qr, a.Tq - 1)) * HD);
    uint4 raw[HD / 16];
    // 4-wave workgroups (small grids, one wave per SIMD) request their Q rows
    // before the table, so the two latencies overlap; with 8 waves the second
    // wave of each SIMD covers it, and the early loads measured slower there.
    if constexpr (NW == 4) {
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) raw[s] = src[2 * s + hf];
    }
    // The table fits only when a workgroup owns bm = 8 * NW query rows (4
    // heads per workgroup, or with WS one head's 32 rows), so a thread fills
    // HD / 16 entries, pairs tid / bm + 8i: with 8 waves pair
    // wave + 8i, with 4 waves 2 wave + hf + 8i. Those indices are uniform over
    // a wave (or half-wave), so the frequencies come by scalar loads, all
    // requested before the first is used.
    constexpr int TBM = 8 * NW;
    constexpr int TPT = (HD / 2) * TBM / NT;
    static_assert((HD / 2) * TBM * sizeof(float2) <= (NW == 8 ? C::STAGE : C::K_BYTES), "table fits");
    const bool table = a.rope && gm.bm == TBM;
    // (the table is shared: with WS it sits in wave 0's K buffer 1)
    float2* cs = reinterpret_cast<float2*>(WS ? LBW(0, 1) : kbuf(1));  // [HD/2][bm]
    // (loaded whether or not the table is built: kernel arguments, always valid)
    double fr[TPT];
    const int pw = NW == 8 ? wave : 2 * wave;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      if constexpr (NW == 8) {
        fr[i] = a.freqs.rev[pw + 8 * i];
      } else {
        const double f0 = a.freqs.rev[pw + 8 * i], f1 = a.freqs.rev[pw + 1 + 8 * i];
        fr[i] = hf ? f1 : f0;
      }
    }
    if (table) {
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        const int e = tid + i * NT;
        float c, sn;
        rope_cos_sin(a.pos0 + tq0 + e % TBM, fr[i], c, sn);
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
    if constexpr (NW == 8) {
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) raw[s] = src[2 * s + hf];
    }
    if (!a.rope) {
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) ws.qf[s] = as_bf16x8(raw[s]);
    } else {
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) ws.qf[s] = rotate(raw[s], qr, 8 * s + 4 * hf);
    }
  }
  // Tile 0 has landed, V buffer 2 is zeroed and no wave still reads the table.
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
  bool pending = !WINDOW && !REV && (!WS || nkt > kt_begin);
  auto step = [&](int kt, auto mask_tag, auto phase_tag, auto set_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int P = decltype(phase_tag)::value;  // walk step % 6
    constexpr int SET = decltype(set_tag)::value;
    unsigned char* cur = kbuf(P);
    unsigned char* prv = vbuf(P + 5);
    const int k0 = kt * BN;
    if constexpr (REV) {
      if (kt > kt_begin) dma.issue(Kg, Vg, kt - 1, a.Tk, kbuf(P + 1), vbuf(P + 1), dwave);
    } else {
      if (kt + 1 < nkt) dma.issue(Kg, Vg, kt + 1, a.Tk, kbuf(P + 1), vbuf(P + 1), dwave);
    }
    // in a masked tile a wave may be past its last visible key (causal) or
    // before its first one (sliding window)
    const int tw0 = a.q_off + qw0;
    const bool run = wave_active && !(MASK && ((CAUSAL && k0 > tw0 + 31) ||
                                               (WINDOW && k0 + BN - 1 < tw0 - a.window + 1)));
    // every key of the tile visible to all 32 rows: before the first row's
    // token, inside the sequence, inside the last row's window
    const bool full = MASK && (!CAUSAL || k0 + BN - 1 <= tw0) && k0 + BN <= a.Tk &&
                      (!WINDOW || k0 >= tw0 + 32 - a.window);
    if (run) {
      f32x16 sa, sb;
      ws.scores((LdsBytes)cur, sa, sb);
      // A wave in its softmax + deferred-product phase gets issue priority
      // over a wave computing scores (measured: fewer cycles per tile).
      __builtin_amdgcn_s_setprio(1);
      ws.template softmax_pv<MASK, SET>(sa, sb, k0, (LdsBytes)prv, full);
      __builtin_amdgcn_s_setprio(0);
      if constexpr (MASK && (WINDOW || REV)) pending = true;
    } else if (MASK && pending) {
      // past the wave's last visible key: settle the owed product (the wave
      // does not run again)
      ws.pv((LdsBytes)prv, ws.pprev);
      pending = false;
    }
    // (with WS only this wave reads and refills its ring: its own wait is enough)
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (!WS) __syncthreads();
  };
  using F = std::integral_constant<bool, false>;
  using M = std::integral_constant<bool, true>;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  using P4 = std::integral_constant<int, 4>;
  using P5 = std::integral_constant<int, 5>;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  // Walk step j uses the buffers named by j % 6 (the rings turn every 3
  // steps with 8 waves, every 6 with 4), and every loop below starts a round
  // of R steps at 0, so each step names its buffers statically. Masked rounds
  // run the masked step, which is also correct for clean tiles.
  constexpr int R = NW == 8 ? 3 : 6;
  int kt = kt_begin;
  auto masked_rounds = [&](int end) __attribute__((always_inline)) {
    while (kt < end) {
      step(kt, M{}, P0{}, S0{});
      if (++kt >= end) break;
      step(kt, M{}, P1{}, S0{});
      if (++kt >= end) break;
      step(kt, M{}, P2{}, S0{});
      if constexpr (NW == 4) {
        if (++kt >= end) break;
        step(kt, M{}, P3{}, S0{});
        if (++kt >= end) break;
        step(kt, M{}, P4{}, S0{});
        if (++kt >= end) break;
        step(kt, M{}, P5{}, S0{});
      }
      ++kt;
    }
  };
  if constexpr (REV) {
    // Step i takes tile nkt-1-i into ring stage i % 3. The masked tiles at the
    // top come first, in whole rounds of the ring (a round that is not all
    // masked runs masked), then the clean tiles. A wave skips the masked tiles
    // past its last token and runs every tile from its first visible one on.
    const int total = nkt - kt_begin;
    const int mend = min(total, (nkt - kc_hi + R - 1) / R * R);
    int i = 0;
    auto masked_rev = [&](int end) __attribute__((always_inline)) {
      while (i < end) {
        step(nkt - 1 - i, M{}, P0{}, S0{});
        if (++i >= end) break;
        step(nkt - 1 - i, M{}, P1{}, S0{});
        if (++i >= end) break;
        step(nkt - 1 - i, M{}, P2{}, S0{});
        if constexpr (NW == 4) {
          if (++i >= end) break;
          step(nkt - 1 - i, M{}, P3{}, S0{});
          if (++i >= end) break;
          step(nkt - 1 - i, M{}, P4{}, S0{});
          if (++i >= end) break;
          step(nkt - 1 - i, M{}, P5{}, S0{});
        }
        ++i;
      }
    };
    masked_rev(mend);
    for (; i + 6 <= total; i += 6) {
      step(nkt - 1 - i, F{}, P0{}, S1{});
      step(nkt - 2 - i, F{}, P1{}, S2{});
      step(nkt - 3 - i, F{}, P2{}, S1{});
      step(nkt - 4 - i, F{}, P3{}, S2{});
      step(nkt - 5 - i, F{}, P4{}, S1{});
      step(nkt - 6 - i, F{}, P5{}, S2{});
    }
    if constexpr (NW == 8) {
      for (; i + 3 <= total; i += 3) {
        step(nkt - 1 - i, F{}, P0{}, S0{});
        step(nkt - 2 - i, F{}, P1{}, S0{});
        step(nkt - 3 - i, F{}, P2{}, S0{});
      }
    }
    // the last clean tiles, fewer than a round (the rounds are at 0 here)
    if (i < total) step(nkt - 1 - i, F{}, P0{}, S0{});
    if (i + 1 < total) step(nkt - 2 - i, F{}, P1{}, S0{});
    if constexpr (NW == 4) {
      if (i + 2 < total) step(nkt - 3 - i, F{}, P2{}, S0{});
      if (i + 3 < total) step(nkt - 4 - i, F{}, P3{}, S0{});
      if (i + 4 < total) step(nkt - 5 - i, F{}, P4{}, S0{});
    }
    // the last step took tile kt_begin = 0, which every row sees; with WS a
    // wave that skipped every tile of its share still owes only the zeros its
    // operands started as
    pending = total > 0;
  } else {
  if constexpr (WINDOW) {
    // tiles at the window's start, up to the first round boundary at or after
    // the first clean tile
    masked_rounds(min(nkt, kt_begin + (kc_lo - kt_begin + R - 1) / R * R));
  }
  if constexpr (WINDOW) {
    if (kt + R <= kc_hi) pending = true;  // every active wave runs a clean tile
  }
  // Clean tiles six per iteration (two turns of the ring): with an even step
  // count the pending probabilities can alternate between two register sets
  // instead of being copied at every step; then three at a time.
  for (; kt + 6 <= kc_hi; kt += 6) {
    step(kt, F{}, P0{}, S1{});
    step(kt + 1, F{}, P1{}, S2{});
    step(kt + 2, F{}, P2{}, S1{});
    step(kt + 3, F{}, P3{}, S2{});
    step(kt + 4, F{}, P4{}, S1{});
    step(kt + 5, F{}, P5{}, S2{});
  }
  if constexpr (NW == 8) {
    for (; kt + 3 <= kc_hi; kt += 3) {
      step(kt, F{}, P0{}, S0{});
      step(kt + 1, F{}, P1{}, S0{});
      step(kt + 2, F{}, P2{}, S0{});
    }
  }
  masked_rounds(nkt);
  }
  // the last tile's V^T product (no DMA is in flight any more)
  if (wave_active && pending) ws.pv((LdsBytes)vbuf((nkt - 1 - kt_begin) % 3), ws.pprev);
  if constexpr (WS) {
    // Every wave leaves its state in its own K buffers (O: HD/2 registers x
    // 64 lanes x 4 bytes, one buffer; the running max and denominator in the
    // other); then each wave merges the four states for a quarter of the head
    // dimensions (accumulator registers wave*HD/8 .. +HD/8 in the order
    // 16 mb + r) and writes that quarter of every row.
    static_assert((HD / 2) * 64 * 4 == C::K_BYTES, "one wave's O fills one buffer");
    {
      float* xo = reinterpret_cast<float*>(LB(0));
      float* xm = reinterpret_cast<float*>(LB(1));
#pragma unroll
      for (int mb = 0; mb < HD / 32; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(mb * 16 + r) * 64 + lane] = ws.oacc[mb][r];
      xm[lane] = ws.m_run;
      xm[64 + lane] = ws.l_run;
    }
    __syncthreads();
    auto xo_of = [&](int w) __attribute__((always_inline)) {
      return reinterpret_cast<const float*>(w == 0 ? LBW(0, 0) : (w == 1 ? LBW(1, 0) : (w == 2 ? LBW(2, 0) : LBW(3, 0))));
    };
    auto xm_of = [&](int w) __attribute__((always_inline)) {
      return reinterpret_cast<const float*>(w == 0 ? LBW(0, 1) : (w == 1 ? LBW(1, 1) : (w == 2 ? LBW(2, 1) : LBW(3, 1))));
    };
    // O and l of each share are relative to that share's own running max
    float mw[4], aw[4];
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = xm_of(w)[lane];
      mx = fmaxf(mx, mw[w]);
    }
    const float mr = mx == -INFINITY ? 0.f : mx;
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      aw[w] = __builtin_amdgcn_exp2f(mw[w] - mr);
      l = fmaf(xm_of(w)[64 + lane], aw[w], l);
    }
    const float l_tot = l + xhalf(l);
    const float inv_l = 1.0f / l_tot;
    constexpr int QR = HD / 8;
    float o[QR];
#pragma unroll
    for (int i = 0; i < QR; ++i) o[i] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* xo = xo_of(w) + wave * QR * 64 + lane;
#pragma unroll
      for (int i = 0; i < QR; ++i) o[i] = fmaf(xo[i * 64], aw[w], o[i]);
    }
    const int qi = qw0 + n;
    if (wave_active && qi < a.Tq) {
      const long orow = (((long)b * a.H + head) * a.Tq + qi) * HD;
#pragma unroll
      for (int g = 0; g < QR / 4; ++g) {
        // registers f .. f+3 hold dims d .. d+3 of the lane's row
        const int f = wave * QR + 4 * g;
        const int d = 32 * (f / 16) + 8 * ((f % 16) / 4) + 4 * hf;
        const float o0 = o[4 * g] * inv_l, o1 = o[4 * g + 1] * inv_l, o2 = o[4 * g + 2] * inv_l, o3 = o[4 * g + 3] * inv_l;
        if constexpr (OUT_BF16) {
          typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + orow + d) =
              u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + orow + d) = make_float4(o0, o1, o2, o3);
        }
      }
      if (wave == 0 && a.lse && hf == 0)
        a.lse[((long)b * a.H + head) * a.Tq + qi] = (mx + log2f(l_tot)) * 0.69314718055994531f;
    }
    return;
  }
  if (!wave_active) return;

  const float l_tot = ws.l_run + xhalf(ws.l_run);
  const float inv_l = 1.0f / l_tot;
  if constexpr (OUT_BF16) {
    // bf16 O leaves through LDS so that every store instruction writes whole
    // rows: the wave puts its 32 rows, in the accumulator layout, into a
    // private slot (8 waves: a quarter of one of the two ring stages the last
    // tile does not occupy; 4 waves: half of a K buffer; no wave reads those
    // any more and no DMA is in flight), then reads them back row-major.
    // 16-byte chunks are XOR-swizzled by row, so neither side has bank
    // conflicts.
    constexpr int RB = 2 * HD;    // bytes of one output row
    constexpr int CPR = RB / 16;  // 16-byte chunks per row
    constexpr int RPI = 64 / CPR; // rows per read-back instruction
    // (lane indices re-derived here, so the compiler does not compute the
    // epilogue's addresses before the loop and hold them through it)
    int el = lane;
    asm volatile("" : "+v"(el));
    const int en = el & 31, ehf = el >> 5;
    LDS unsigned char* slot;
    if constexpr (NW == 8) {
      const int p_last = (nkt - 1 - kt_begin) % 3;
      unsigned char* fs = (wave < 4) ? (p_last == 0 ? LB(1) : LB(0)) : (p_last == 2 ? LB(1) : LB(2));
      slot = (LDS unsigned char*)(fs + (wave & 3) * (C::STAGE / 4));
    } else {
      slot = (LDS unsigned char*)(kbuf(wave >> 1) + (wave & 1) * (C::K_BYTES / 2));
    }
#pragma unroll
    for (int mb = 0; mb < HD / 32; ++mb) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = 4 * mb + g4;  // chunk of d = 32mb + 8g4 .. +7; this lane holds half 'ehf' of it
        LDS unsigned char* dst = slot + en * RB + ((c ^ (en % CPR)) * 16) + 8 * ehf;
        const float o0 = ws.oacc[mb][4 * g4 + 0] * inv_l, o1 = ws.oacc[mb][4 * g4 + 1] * inv_l;
        const float o2 = ws.oacc[mb][4 * g4 + 2] * inv_l, o3 = ws.oacc[mb][4 * g4 + 3] * inv_l;
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<LDS u32x2*>(dst) = u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const long obase = ((long)b * a.H + head) * a.Tq + qw0;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + el / CPR, c = el % CPR;
      const u32x4 v = *reinterpret_cast<const LDS u32x4*>(slot + r * RB + ((c ^ (r % CPR)) * 16));
      if (qw0 + r < a.Tq)
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + (obase + r) * HD + c * 8) = v;
    }
  } else {
    const int qi = qw0 + n;
    if (qi < a.Tq) {
      const long orow = (((long)b * a.H + head) * a.Tq + qi) * HD;
#pragma unroll
      for (int mb = 0; mb < HD / 32; ++mb) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = 32 * mb + 8 * g4 + 4 * hf;
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + orow + d) =
              make_float4(ws.oacc[mb][4 * g4 + 0] * inv_l, ws.oacc[mb][4 * g4 + 1] * inv_l,
                          ws.oacc[mb][4 * g4 + 2] * inv_l, ws.oacc[mb][4 * g4 + 3] * inv_l);
        }
      }
    }
  }
  const int qi = qw0 + n;  // query row
  if (qi >= a.Tq) return;
  if (a.lse && hf == 0) a.lse[((long)b * a.H + head) * a.Tq + qi] = (ws.m_run + log2f(l_tot)) * 0.69314718055994531f;
#undef LB
#undef LBW
}

// nw = 0: the wave-split grid (one head and 32 query rows per workgroup)
GridMap make_grid(const PrefillArgs& a, int nw) {
  GridMap gm;
  gm.hpw = nw == 0 ? 1 : (a.group % 4 == 0) ? 4 : (a.group % 2 == 0 ? 2 : 1);
  gm.hchunks = a.group / gm.hpw;
  gm.bm = nw == 0 ? 32 : 32 * (nw / gm.hpw);
  gm.nqb = (a.Tq + gm.bm - 1) / gm.bm;
  gm.units = a.B * a.KV * gm.hchunks;
  gm.xcd_aware = (gm.units % 8) == 0;
  // units per XCD group: their K/V (2 * Tk * hd * 2 bytes each) within 4 MiB,
  // the L2 of one XCD, but at least 32 workgroups (one per CU of the XCD)
  const long unit_bytes = 4L * a.Tk * a.hd;
  const int upx = gm.units >> 3;
  int ug = (int)max(1L, (4L << 20) / unit_bytes);
  while (ug * gm.nqb < 32 && ug < upx) ++ug;
  gm.ugroup = max(1, min(ug, upx));
  return gm;
}

template <int HD, int NW, bool ALIBI, bool CAUSAL, bool WINDOW, bool WS>
void launch_out(const PrefillArgs& a, const GridMap& gm, dim3 grid, hipStream_t s) {
  if (a.out_bf16) {
    hipLaunchKernelGGL((prefill_mfma_kernel<HD, NW, ALIBI, CAUSAL, true, WINDOW, WS>), grid, dim3(NW * 64), 0, s, a, gm);
  } else {
    hipLaunchKernelGGL((prefill_mfma_kernel<HD, NW, ALIBI, CAUSAL, false, WINDOW, WS>), grid, dim3(NW * 64), 0, s, a,
                       gm);
  }
}

// The sliding window is a separate instance (causal only), so the plain
// kernels carry none of its masking or tile-skipping code.
template <int HD, int NW, bool WS>
void launch_hd(const PrefillArgs& a, const GridMap& gm, dim3 grid, hipStream_t s) {
  if (a.alibi) {
    if (a.window > 0) launch_out<HD, NW, true, true, true, WS>(a, gm, grid, s);
    else if (a.causal) launch_out<HD, NW, true, true, false, WS>(a, gm, grid, s);
    else launch_out<HD, NW, true, false, false, WS>(a, gm, grid, s);
  } else {
    if (a.window > 0) launch_out<HD, NW, false, true, true, WS>(a, gm, grid, s);
    else if (a.causal) launch_out<HD, NW, false, true, false, WS>(a, gm, grid, s);
    else launch_out<HD, NW, false, false, false, WS>(a, gm, grid, s);
  }
}

// Compute units of the current device (looked up once per device).
int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
  }
  return cus[dev];
}

// Waves per workgroup: 8 unless the 8-wave grid leaves compute units without
// a workgroup. ATTN_PREFILL_WAVES=4 or 8 forces one (for tests).
int pick_waves(const PrefillArgs& a) {
  if (const char* e = getenv("ATTN_PREFILL_WAVES")) {
    if (e[0] == '4' && e[1] == 0) return 4;
    if (e[0] == '8' && e[1] == 0) return 8;
  }
  const GridMap gm = make_grid(a, 8);
  return (long)gm.units * gm.nqb < device_cus() ? 4 : 8;
}

// Wave-split workgroups (head size 64: four rings fill the 160 KiB of LDS)
// when the 4-wave grid leaves compute units idle, the wave-split grid fits
// the compute units and some block walks more than four key tiles.
// ATTN_PREFILL_WSPLIT=0 or 1 forces the choice at head size 64 (for tests).
bool pick_wsplit(const PrefillArgs& a) {
  if (a.hd != 64) return false;
  if (const char* e = getenv("ATTN_PREFILL_WSPLIT")) {
    if (e[0] == '0' && e[1] == 0) return false;
    if (e[0] == '1' && e[1] == 0) return true;
  }
  if (getenv("ATTN_PREFILL_WAVES")) return false;  // a forced workgroup size keeps its kernel
  const GridMap g4 = make_grid(a, 4), gw = make_grid(a, 0);
  const int last = a.causal ? a.q_off + a.Tq - 1 : a.Tk - 1;  // the last key any row sees
  return (long)g4.units * g4.nqb < device_cus() && (long)gw.units * gw.nqb <= device_cus() && last >= 4 * BN;
}

}  // namespace

bool prefill_mfma_supported(const PrefillArgs& a, int bf16) {
  if (!bf16 || (a.hd != 64 && a.hd != 128)) return false;
  if ((long)a.Tk * a.hd * 2 >= (1L << 31)) return false;  // buffer descriptors hold 32-bit sizes
  const GridMap gm = make_grid(a, 0);  // (the wave-split grid is the largest)
  return (long)gm.units * gm.nqb < (1L << 31);
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s) {
  if (pick_wsplit(a)) {
    const GridMap gm = make_grid(a, 0);
    launch_hd<64, 4, true>(a, gm, dim3((unsigned)(gm.units * gm.nqb)), s);
    return hipGetLastError();
  }
  const int nw = pick_waves(a);
  const GridMap gm = make_grid(a, nw);
  const dim3 grid((unsigned)(gm.units * gm.nqb));
  if (a.hd == 128) {
    if (nw == 8) launch_hd<128, 8, false>(a, gm, grid, s);
    else launch_hd<128, 4, false>(a, gm, grid, s);
  } else {
    if (nw == 8) launch_hd<64, 8, false>(a, gm, grid, s);
    else launch_hd<64, 4, false>(a, gm, grid, s);
  }
  return hipGetLastError();
}

}  // namespace attn
