// Latent-attention decode (gfx950).
//
// Exercise 5 of "Write attention from scratch": every token keeps one latent
// vector c_j (d_c numbers shared by all heads); head h's key and value are
// c_j W_uk[h] and c_j W_uv[h]. Folding the key up-projection into the query,
// q~_h = W_uk[h] q_h, makes the score <q~_h, c_j>/sqrt(hd), and the output is
// (sum_j p_hj c_j) W_uv[h]. So a decode step is
//   1. fold:   q~[b, h] = W_uk[h] q[b, h]                      (small GEMM)
//   2. split:  attention of the H folded queries over the latent cache, one
//              latent row serving as both key and value, split-KV partials
//   3. merge:  log-sum-exp merge of the partials -> o~[b, h] (d_c numbers)
//   4. up:     out[b, h] = o~[b, h] W_uv[h]                    (small GEMM)
// with the new token's latent written to cache slot L (its position) and
// attended there. No rotary embedding on this path: a rotation of the keys
// would not commute with the fold.
//
// The split kernel is where the bytes are: the cache is read once per step for
// all heads. Each wave streams 16-key tiles of the latent cache into its own
// LDS rows by LDS-DMA, one tile landing while it computes on the previous one,
// and waits only for its own DMA (no barrier while streaming); workgroups are
// one wave, so four of them share a CU and their loads overlap. The 16 heads
// of a head block are the columns of S^T = C Q~^T (16x16x32 MFMA over d_c);
// P^T comes out of the accumulators in the B-operand layout of the 16x16x16
// MFMA that accumulates O~^T += C^T P^T, whose A operand (16 latent dims x 4
// keys per lane group) is one transposing LDS read.
#include <type_traits>

#include "mfma_tile.h"

namespace attn {

namespace {

using namespace tile;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2eL = 1.4426950408889634f;
constexpr float kLn2L = 0.69314718055994531f;
constexpr int kLW = 1;   // waves per split workgroup (16 keys of each tile per wave)
constexpr int kNST = 2;  // LDS stages (tiles in flight + the one computed on)

__device__ __forceinline__ bool lat_bad_len(int L, int Lmax) { return L < 0 || L >= Lmax; }

// Swizzle of the 16-byte chunk index of latent row r (rows are 2*d_c bytes,
// a multiple of 256, so every row starts at bank 0). Row reads: 16 lanes read
// one logical chunk of rows 16w .. 16w+15 -> 16 different slots over row bits
// 0..3, bit 0 from row bit 0. Transposing reads: 32 lanes read rows
// 16w + (0..7) x 32 bytes -> bits 1..3 take 8 values over row bits 0..2.
__host__ __device__ constexpr int lat_swz(int r) {
  return (r & 1) | ((((r >> 0) ^ (r >> 3)) & 1) << 1) | (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 3);
}
template <int DC>
__host__ __device__ constexpr int lat_off(int r, int c) { return r * DC * 2 + ((c ^ lat_swz(r)) << 4); }

// ----------------------------------------------------------------- 1. fold
// Per head a small GEMM, Q~_h (B x d_c) = Q_h (B x hd) W_uk[h]^T (hd x d_c),
// on the 16x16x32 bf16 MFMA (fp32 accumulation; the bf16 products are exact).
// Grid (H, ceil(B/16), d_c/64), 4 waves: wave w computes the 16 x 16 block of
// batch rows 16*blockIdx.y .., latent dims 64*blockIdx.z + 16w ... Both
// operands come straight from memory in the MFMA layout: lane (n, g) of
// k-step s holds dims 32s + 8g .. +7 of query row n (A) and of W_uk row n (B),
// 16 contiguous bytes each, so all loads of a wave are in flight at once.
// The split kernel's work list, built by one workgroup of the fold: the
// active (sequence, split) pairs, sequence by sequence, as b * kLatentMaxSplits
// + split, followed by their count. Split workgroup i takes pair i, so the
// workgroups that do work are dispatched first and the surplus ones (the grid
// is sized for every sequence at Lmax) exit at the end.
__device__ void latent_build_items(const LatentArgs& a) {
  __shared__ int part[256];
  const int tid = threadIdx.x;
  const int per = (a.B + 255) / 256;
  const int b0 = min(a.B, tid * per), b1 = min(a.B, b0 + per);
  auto nsplits = [&](int b) {
    const int L = a.lens[b];
    return lat_bad_len(L, a.Lmax) ? 0 : (L + 1 + a.split - 1) / a.split;
  };
  int cnt = 0;
  for (int b = b0; b < b1; ++b) cnt += nsplits(b);
  part[tid] = cnt;
  __syncthreads();
  // inclusive scan of the 256 counts (Hillis-Steele)
  for (int o = 1; o < 256; o <<= 1) {
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int at = part[tid] - cnt;
  for (int b = b0; b < b1; ++b) {
    const int ns = nsplits(b);
    for (int sp = 0; sp < ns; ++sp) a.items[at++] = b * kLatentMaxSplits + sp;
  }
  if (tid == 255) a.items[a.B * a.nsplit] = part[255];
}

template <int HD>
__global__ __launch_bounds__(256) void latent_fold_kernel(LatentArgs a) {
  constexpr int NK = HD / 32;
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) latent_build_items(a);
  const int h = blockIdx.x, lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int wave = threadIdx.x >> 6;
  const int b0 = blockIdx.y * 16, c0 = blockIdx.z * 64 + 16 * wave;
  const bool brow = b0 + n < a.B;
  const uint4* qrow = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                                     ((long)(brow ? b0 + n : 0) * a.H + h) * HD);
  const uint4* wrow = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.w_uk) +
                                                     ((long)h * a.dc + c0 + n) * HD);
  bf16x8 qa[NK], wb[NK];
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    qa[s] = as_bf16x8(brow ? qrow[4 * s + g] : make_uint4(0, 0, 0, 0));
    wb[s] = as_bf16x8(wrow[4 * s + g]);
  }
  f32x4 acc = f32x4{};
#pragma unroll
  for (int s = 0; s < NK; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], wb[s], acc, 0, 0, 0);
  // lane (n, g) holds batch rows b0 + 4g + i, latent dim c0 + n
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int bb = b0 + 4 * g + i;
    if (bb < a.B) a.qt[((long)bb * a.H + h) * a.dc + c0 + n] = f32_to_bf16_bits(acc[i]);
  }
}

// ---------------------------------------------------------------- 2. split
// vmcnt wait immediate (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt and
// lgkmcnt left at their maxima): wait until at most n vector-memory operations
// of this wave are outstanding.
template <int N>
constexpr int vmcnt_imm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  return (N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14);
}

constexpr int lgkm0_imm() { return 15 | (7 << 4) | (0 << 8) | (3 << 14); }  // lgkmcnt(0) only

template <int DC, int LW, int NST>
__global__ __launch_bounds__(LW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void latent_split_kernel(LatentArgs a) {
  constexpr int LT = 16 * LW;              // keys per tile (16 per wave)
  constexpr int ROW = DC * 2;              // bytes per latent row
  constexpr int STAGE = LT * ROW;          // one tile
  constexpr int PW = 16 * ROW / 1024;      // 1 KiB LDS-DMA instructions per wave per tile
  constexpr int NS = DC / 32;              // k-steps of S^T
  constexpr int NB = DC / 16;              // 16-dim blocks of O~^T
  static_assert(NST >= 2 && NST <= 4 && (NST - 1) * PW < 64, "stage count");
  static_assert(kLatentSplit % LT == 0, "a split is whole tiles");
  // the stages, each its own LDS object (named statically at every use, so
  // the compiler never waits on a DMA into one stage before reading another)
  __shared__ __attribute__((aligned(16))) unsigned char s0[STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char s1[STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char s2[NST > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) unsigned char s3[NST > 3 ? STAGE : 16];
  __shared__ float mer_m[LW][16];
  __shared__ float mer_l[LW][16];

  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // grid (B * nsplit, hblocks): workgroup i takes the i-th active (sequence, split) pair
  const int nitems = a.items[a.B * a.nsplit];
  if ((int)blockIdx.x >= nitems) return;
  const int item = a.items[blockIdx.x];
  const int b = item / kLatentMaxSplits, sp = item % kLatentMaxSplits, hb = blockIdx.y;
  const int L = a.lens[b];
  if (lat_bad_len(L, a.Lmax)) return;
  const int nk = L + 1;
  const int k0 = sp * a.split;
  if (k0 >= nk) return;
  const int k1 = min(nk, k0 + a.split);
  const int ntile = (k1 - k0 + LT - 1) / LT;
  const int head = hb * 16 + n;
  const bool qcol = head < a.H;

  // Q~^T B operand (column n = head hb*16 + n, k-step s holds dims 32s + 8g
  // .. +7) and the new latent, loaded before the first tiles so that their
  // waits do not cover the tiles' DMA
  bf16x8 qf[NS];
  {
    const uint4* src = reinterpret_cast<const uint4*>(a.qt + ((long)b * a.H + (qcol ? head : 0)) * DC);
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = as_bf16x8(qcol ? src[4 * s + g] : make_uint4(0, 0, 0, 0));
  }
  // The workgroup holding slot L writes the new latent there; the wave whose
  // keys include L patches that row of its LDS tile once the tile has landed.
  const bool own_slot = L >= k0 && L < k1;
  uint4 cnew = make_uint4(0, 0, 0, 0);
  if (own_slot && lane < DC / 8) {
    cnew = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.c_new) + (long)b * DC)[lane];
    if (wave == 0)
      reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.c_cache) + ((long)b * a.Lmax + L) * DC)[lane] = cnew;
  }

  const unsigned char* Cg = reinterpret_cast<const unsigned char*>(a.c_cache) + (long)b * a.Lmax * ROW;
  // (The loads carry the non-temporal policy: the cache is read once per step.)
  // Wave w's part of tile t: rows 16w .. 16w+15, which only wave w reads, so
  // a wave waits for its own DMA and no barrier is needed while streaming.
  // Tiles of one split end before the next split starts; the descriptor ends
  // at the sequence end, so rows past it arrive as zeros. A tile past the
  // split's last one gets an empty descriptor (no memory is read), so every
  // step issues the same number of DMA instructions and the waits count
  // exactly.
  auto issue = [&](int t, unsigned char* stage) __attribute__((always_inline)) {
    const int ts = k0 + t * LT;
    const int rows = t < ntile ? nk - ts : 0;
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t r = make_rsrc(Cg + (long)min(ts, nk) * ROW, rows * ROW);
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      // lane's 16 bytes of instruction q land at LDS byte 1024q + 16 lane: row
      // r, physical chunk pc, which holds logical chunk pc ^ swz(r)
      const int p = 1024 * (wave * PW + i) + 16 * lane;
      const int row = p / ROW, pc = (p % ROW) / 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)(stage + 1024 * (wave * PW + i)), 16,
                                               row * ROW + ((pc ^ lat_swz(row)) << 4), 0, 0, 2);
    }
#endif
  };
  issue(0, s0);
  if constexpr (NST > 2) issue(1, s1);
  if constexpr (NST > 3) issue(2, s2);

  const float c2 = a.scale_log2;
  const float slope2 = (a.alibi && qcol) ? alibi_slope(a.alibi, head, a.H) * kLog2eL : 0.f;
  // transposing-read offsets: lane (li, g) reads row 16*wave + 4g + li/4, dims 16db + 4(li%4) .. +3
  const int li = lane & 15;
  const int trow = 16 * wave + 4 * g + (li >> 2);
  const int tcol = 4 * (li & 3);
  const int srow = 16 * wave + n;  // row read for S^T (natural key order)
  // The swizzle is 4 bits, so a read's byte offset is a per-lane base that
  // depends on the low bits of the chunk index plus 256 x the rest: row reads
  // of chunk 4st + g use base sbase[st & 3] + 256 (st >> 2), transposing reads
  // of dim block db use tbase[db & 7] + 256 (db >> 3) (instruction offsets).
  int sbase[4], tbase[8];
  {
    const int sw = lat_swz(srow), tw = lat_swz(trow);
#pragma unroll
    for (int m = 0; m < 4; ++m) sbase[m] = srow * ROW + 64 * (m ^ (sw >> 2)) + 16 * (g ^ (sw & 3));
#pragma unroll
    for (int m = 0; m < 8; ++m)
      tbase[m] = trow * ROW + 32 * (m ^ (tw >> 1)) + 16 * ((tcol >> 3) ^ (tw & 1)) + 2 * (tcol & 7);
  }
  static_assert(lat_off<512>(37, 4 * 9 + 2) == 37 * 1024 + 64 * (1 ^ (lat_swz(37) >> 2)) + 16 * (2 ^ (lat_swz(37) & 3)) + 256 * 2,
                "row-read base decomposition");
  static_assert(lat_off<512>(21, (16 * 11 + 8) >> 3) + 0 ==
                    21 * 1024 + 32 * (3 ^ (lat_swz(21) >> 1)) + 16 * (1 ^ (lat_swz(21) & 1)) + 256 * 1,
                "transposing-read base decomposition");

  f32x4 oacc[NB];
#pragma unroll
  for (int db = 0; db < NB; ++db) oacc[db] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;

  // Step t: issue tile t+NST-1 into the stage of tile t-1 (this wave's reads
  // of it ended with the step), wait for this wave's DMA of tile t (NST-1
  // tiles' instructions may stay in flight), compute on it.
  auto step = [&](int t, auto par) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    constexpr int PN = (P + NST - 1) % NST;
    unsigned char* cur = P == 0 ? s0 : (P == 1 ? s1 : (P == 2 ? s2 : s3));
    unsigned char* nxt = PN == 0 ? s0 : (PN == 1 ? s1 : (PN == 2 ? s2 : s3));
    issue(t + NST - 1, nxt);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<(NST - 1) * PW>());
    const int ts = k0 + t * LT;
    const int kw = ts + 16 * wave;  // the wave's first key
    if (kw < k1) {
      LdsBytes tile = (LdsBytes)cur;
      if (own_slot && L >= kw && L < kw + 16 && lane < DC / 8) {
        const int r = L - ts;
        *reinterpret_cast<LDS u32x4*>((LDS unsigned char*)cur + lat_off<DC>(r, lane)) = __builtin_bit_cast(u32x4, cnew);
      }
      // S^T: every row read issued first, two independent accumulator chains
      bf16x8 av[NS];
#pragma unroll
      for (int st = 0; st < NS; ++st)
        av[st] = *reinterpret_cast<const LDS bf16x8*>(tile + sbase[st & 3] + 256 * (st >> 2));
      f32x4 sa = f32x4{}, sb = f32x4{};
#pragma unroll
      for (int st = 0; st < NS; st += 2) {
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[st], qf[st], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[st + 1], qf[st + 1], sb, 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, NS, 0);  // the NS row reads,
      __builtin_amdgcn_sched_group_barrier(0x008, NS, 0);  // then the NS MFMAs
      // the transposing reads of the P V step do not depend on S: issue them
      // now so that they land under the softmax
      i16x4 tv[NB];
#pragma unroll
      for (int db = 0; db < NB; ++db)
        tv[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS i16x4*)((LDS unsigned char*)cur + tbase[db & 7] + 256 * (db >> 3)));
      const f32x4 s = sa + sb;
      // register i: key kw + 4g + i, column = head
      float x[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kw + 4 * g + i;
        float v = s[i] * c2;
        if (a.alibi) v = fmaf(slope2, (float)(key - L), v);
        v = key < k1 ? v : -INFINITY;
        x[i] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // lazy rescale: keep the running max unless the tile's exceeds it by more
      // than 2^8 (numerator and denominator share the max, so the ratio holds)
      const bool bump = mx > m_run + 8.f;
      const float m_use = bump ? mx : m_run;
      float p[4], lsum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(x[i] - m_use);
        lsum += p[i];
      }
      if (__any(bump)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NB; ++db) oacc[db] *= alpha;
      }
      m_run = m_use;
      l_run += lsum;
      const bf16x4 pb = __builtin_bit_cast(bf16x4, make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])));
#pragma unroll
      for (int db = 0; db < NB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, tv[db]), pb, oacc[db], 0, 0, 0);
    }
    // this wave's reads of the stage are done before its next DMA overwrites it
    __builtin_amdgcn_s_waitcnt(lgkm0_imm());
  };
  // NST steps per iteration, so each names its stage statically. A step past
  // the split's last tile finds an empty tile and computes nothing
  // (its keys are at or past the split end k1); its DMA reads no memory. The
  // loop keeps the code small: fully unrolled over a split, the kernel was
  // about ten times the instruction cache and ran fetch-bound.
  for (int t = 0; t < ntile; t += NST) {
    step(t, std::integral_constant<int, 0>{});
    step(t + 1, std::integral_constant<int, 1>{});
    if constexpr (NST > 2) step(t + 2, std::integral_constant<int, 2>{});
    if constexpr (NST > 3) step(t + 3, std::integral_constant<int, 3>{});
  }
  __builtin_amdgcn_s_waitcnt(0);  // the empty tail tiles issued past the end

  float l_col = l_run + __shfl_xor(l_run, 16);
  l_col += __shfl_xor(l_col, 32);
  const int ncol = min(16, a.H - hb * 16);
  if constexpr (LW == 1) {
    // one wave: its state is the partial
    if (qcol) {
      const long pidx = ((long)b * a.H + head) * a.nsplit + sp;
#pragma unroll
      for (int db = 0; db < NB; ++db)
        *reinterpret_cast<float4*>(a.part_o + pidx * DC + 16 * db + 4 * g) =
            make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
      if (g == 0) a.part_ml[pidx] = make_float2(m_run, l_col);
    }
    (void)ncol;
  } else {
    // ---- merge the waves: per column, M = max_w m_w, weights 2^(m_w - M)
    __syncthreads();  // every wave is done with the stages
    if (g == 0) {
      mer_m[wave][n] = m_run;
      mer_l[wave][n] = l_col;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < LW; ++w) M = fmaxf(M, mer_m[w][n]);
    const float wgt = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
    // wave w's [16][DC] fp32 (64 * DC bytes) goes to stage w / (LW/2) at
    // offset (w % (LW/2)) * 64 * DC: a stage holds LW/2 of them
    constexpr int WPS = LW / 2;
    static_assert(WPS * 64 * DC == STAGE, "two stages hold the waves' outputs");
    float* ob = reinterpret_cast<float*>((wave < WPS ? s0 : s1) + (wave % WPS) * 64 * DC);
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      const int d = 16 * db + 4 * g;
      *reinterpret_cast<float4*>(ob + n * DC + d) =
          make_float4(oacc[db][0] * wgt, oacc[db][1] * wgt, oacc[db][2] * wgt, oacc[db][3] * wgt);
    }
    __syncthreads();
    for (int e = tid; e < ncol * DC; e += LW * 64) {
      const int col = e / DC, d = e % DC;
      const int i = col * DC + d;
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < LW; ++w)
        o += reinterpret_cast<const float*>((w < WPS ? s0 : s1) + (w % WPS) * 64 * DC)[i];
      const long pidx = ((long)b * a.H + hb * 16 + col) * a.nsplit + sp;
      a.part_o[pidx * DC + d] = o;
      if (d == 0) {
        float Mc = -INFINITY;
#pragma unroll
        for (int w = 0; w < LW; ++w) Mc = fmaxf(Mc, mer_m[w][col]);
        float lt = 0.f;
#pragma unroll
        for (int w = 0; w < LW; ++w) {
          const float mw = mer_m[w][col];
          lt += (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - Mc) * mer_l[w][col];
        }
        a.part_ml[pidx] = make_float2(Mc, lt);
      }
    }
  }
}

// ---------------------------------------------------------------- 3. merge
// One (b, h) per 256-thread workgroup: the first wave finds the split weights
// (lanes over splits), then o~[b, h, d] = sum_s w_s O_s[d] / sum_s w_s l_s
// (fp32, workspace) with each thread on DC/256 dims, and the lse.
template <int DC>
__global__ __launch_bounds__(256) void latent_merge_kernel(LatentArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = a.lens[b];
  float* ot = a.ot + ((long)b * a.H + h) * DC;
  if (lat_bad_len(L, a.Lmax)) {
    for (int d = tid; d < DC; d += 256) ot[d] = __builtin_nanf("");
    if (a.lse && tid == 0) a.lse[(long)b * a.H + h] = __builtin_nanf("");
    return;
  }
  const int ns = (L + 1 + a.split - 1) / a.split;  // <= kLatentMaxSplits (host check)
  const long p0 = ((long)b * a.H + h) * a.nsplit;
  __shared__ float wsh[kLatentMaxSplits];
  __shared__ float red[2];
  if (tid < 64) {
    float M = -INFINITY;
    for (int s = tid; s < ns; s += 64) M = fmaxf(M, a.part_ml[p0 + s].x);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float den = 0.f;
    for (int s = tid; s < ns; s += 64) {
      const float2 ml = a.part_ml[p0 + s];
      const float w = exp2f(ml.x - M);
      wsh[s] = w;
      den = fmaf(w, ml.y, den);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o);
    if (tid == 0) {
      red[0] = den;
      red[1] = M;
    }
  }
  __syncthreads();
  const float inv = 1.f / red[0];
  constexpr int PT = DC / 256;  // dims per thread
  float o[PT];
#pragma unroll
  for (int k = 0; k < PT; ++k) o[k] = 0.f;
#pragma unroll 4
  for (int s = 0; s < ns; ++s) {
    const float w = wsh[s];
#pragma unroll
    for (int k = 0; k < PT; ++k) o[k] = fmaf(w, a.part_o[(p0 + s) * DC + tid + 256 * k], o[k]);
  }
#pragma unroll
  for (int k = 0; k < PT; ++k) ot[tid + 256 * k] = o[k] * inv;
  if (a.lse && tid == 0) a.lse[(long)b * a.H + h] = (red[1] + log2f(red[0])) * kLn2L;
}

// ------------------------------------------------------------------- 4. up
// out[b, h, j] = sum_c o~[b, h, c] W_uv[h][c][j] on the fp32 matrix core
// (v_mfma_f32_16x16x4f32: the fp32 latents times the bf16 weights widened to
// fp32, exact products, fp32 sums). Grid (H, ceil(B/16), hd/64), 4 waves: the
// workgroup owns 16 batch rows x 64 output dims of head h, wave w sums the
// latent dims [w DC/4, (w+1) DC/4) and the four partial tiles add through LDS.
// The order of the sum is free, so the operands are laid out for contiguous
// loads: in step s lane group g takes latent dim c = cw + NST*g + s (a lane's
// o~ values are one contiguous run), and column n of MFMA block jb is output
// dim 4n + jb (a lane's 4 weights of a step are 8 contiguous bytes).
template <int HD, int DC>
__global__ __launch_bounds__(256) void latent_up_kernel(LatentArgs a) {
  constexpr int CW = DC / 4;    // latent dims per wave
  constexpr int NST = CW / 4;   // MFMA steps per wave (4 dims each, one per lane group)
  const int h = blockIdx.x, b0 = blockIdx.y * 16, j0 = blockIdx.z * 64;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int wave = tid >> 6;
  const int c0 = wave * CW + NST * g;  // this lane's first latent dim
  const bool row_ok = b0 + n < a.B;
  // A operand: o~[b0 + n, h, c0 .. c0 + NST - 1] (zeros for rows past B)
  // (a row past B reads row B-1 and is zeroed after the load: no branch, so
  // every load of the lane is in flight before the first MFMA waits)
  float4 a4[NST / 4];
  {
    const float4* src = reinterpret_cast<const float4*>(a.ot + ((long)min(b0 + n, a.B - 1) * a.H + h) * DC + c0);
#pragma unroll
    for (int k = 0; k < NST / 4; ++k) a4[k] = src[k];
  }
  // B operand: W_uv[h][c0 + s][j0 + 4n .. + 3], 8 bytes per step
  uint2 wv[NST];
  {
    const uint16_t* w = reinterpret_cast<const uint16_t*>(a.w_uv) + ((long)h * DC + c0) * HD + j0 + 4 * n;
#pragma unroll
    for (int s = 0; s < NST; ++s) wv[s] = *reinterpret_cast<const uint2*>(w + (long)s * HD);
  }
  __builtin_amdgcn_sched_barrier(0);
  float av[NST];
#pragma unroll
  for (int k = 0; k < NST / 4; ++k) {
    av[4 * k] = row_ok ? a4[k].x : 0.f;
    av[4 * k + 1] = row_ok ? a4[k].y : 0.f;
    av[4 * k + 2] = row_ok ? a4[k].z : 0.f;
    av[4 * k + 3] = row_ok ? a4[k].w : 0.f;
  }
  f32x4 acc[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    const float wf[4] = {bf16_bits_to_f32(wv[s].x & 0xffffu), bf16_bits_to_f32(wv[s].x >> 16),
                         bf16_bits_to_f32(wv[s].y & 0xffffu), bf16_bits_to_f32(wv[s].y >> 16)};
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) acc[jb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], wf[jb], acc[jb], 0, 0, 0);
  }
  // lane (n, g) holds rows 4g + r, output dims 4n + jb: add the 4 waves' tiles
  __shared__ float red[4][16][65];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][4 * g + r][4 * n + jb] = acc[jb][r];
  __syncthreads();
#pragma unroll
  for (int e = tid; e < 16 * 64; e += 256) {
    const int r = e >> 6, j = e & 63;
    if (b0 + r >= a.B) continue;
    const float sum = red[0][r][j] + red[1][r][j] + red[2][r][j] + red[3][r][j];
    const long o = ((long)(b0 + r) * a.H + h) * HD + j0 + j;
    if (a.out_bf16) {
      reinterpret_cast<uint16_t*>(a.out)[o] = f32_to_bf16_bits(sum);
    } else {
      reinterpret_cast<float*>(a.out)[o] = sum;
    }
  }
}

template <int HD, int DC>
hipError_t launch_latent_hd(const LatentArgs& a, hipStream_t s, const TimingHook& tm) {
  hipError_t e;
  hipLaunchKernelGGL((latent_fold_kernel<HD>), dim3(a.H, (a.B + 15) / 16, DC / 64), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = tm.before(s)) != hipSuccess) return e;
  hipLaunchKernelGGL((latent_split_kernel<DC, kLW, kNST>), dim3(a.B * a.nsplit, a.hblocks), dim3(kLW * 64), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = tm.after(s)) != hipSuccess) return e;
  hipLaunchKernelGGL((latent_merge_kernel<DC>), dim3(a.H, a.B), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((latent_up_kernel<HD, DC>), dim3(a.H, (a.B + 15) / 16, HD / 64), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_latent(const LatentArgs& a, hipStream_t s, const TimingHook& tm) {
  if (a.hd == 128) {
    return a.dc == 512 ? launch_latent_hd<128, 512>(a, s, tm) : launch_latent_hd<128, 256>(a, s, tm);
  }
  return a.dc == 512 ? launch_latent_hd<64, 512>(a, s, tm) : launch_latent_hd<64, 256>(a, s, tm);
}

}  // namespace attn
