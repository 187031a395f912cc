// The projections either side of attention ("Building Grouped-Query Attention
// with RoPE and Flash Attention from Scratch", Architecture Overview and
// Step 4): the fused QKV input projection, whose epilogue applies the rotary
// embedding to q and k, splits the heads into [B, heads, T, hd] and can write
// k and v straight into a KV cache, and the output projection, whose operand
// loads gather the heads of [B, H, T, hd] back into rows of H*hd.
//
// Both are C[M, N] = A[M, K] W[N, K]^T with both operands contiguous along K,
// the layout the matrix-core operands want: a lane's 8 consecutive K values
// are 16 contiguous bytes of one row.
//
// Kernel
//   * A workgroup of 4 waves computes a 256 x 256 tile of C; wave (wm, wn)
//     owns a 128 x 128 quarter as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16
//     (fp32 accumulators, 256 per lane).
//   * K advances in blocks of 64: the 256 x 64 slices of A and W go global ->
//     LDS by LDS-DMA (buffer loads that write LDS directly) into two stages,
//     block k+1 landing while block k is multiplied. Rows are 128 bytes with
//     16-byte chunks XOR-swizzled by (row >> 1) & 7, which keeps the operand
//     reads (16 lanes reading one chunk of 16 consecutive rows) free of bank
//     conflicts.
//   * Rows past M (or N) sit past the end of their buffer descriptor and read
//     as zeros; their results are never stored.
//   * Tile order: workgroups are dispatched round-robin over the 8 XCDs, so
//     workgroup id i is given tile number (i mod 8) * tiles/8 + i / 8 (each XCD
//     walks a contiguous range of tiles), and tile numbers run down groups of
//     4 row-tiles before moving to the next column: the workgroups resident
//     on one XCD share a few A and W slices in its L2.
#include "mfma_tile.h"
#include "proj_internal.h"

namespace attn {

namespace {

using namespace tile;

constexpr int GBM = 256;                   // tile rows (M)
constexpr int GBN = 256;                   // tile columns (N)
constexpr int GBK = 64;                    // K block
constexpr int GTILE = GBM * GBK * 2;       // bytes of one operand slice in LDS (32 KiB)
constexpr int GPW = GTILE / 1024 / 4;      // 1 KiB LDS-DMA instructions per wave per operand slice
constexpr int GROUP_M = 4;                 // row-tiles per group of the tile order
constexpr unsigned kOob = 0x7fffff00u;     // a voffset past every descriptor: the load returns zeros

static_assert(GBN == GBM, "one slice shape for A and W");

// Chunk swizzle of a 128-byte row (the 64-dim K tile's, measured conflict-free
// for this read pattern).
__host__ __device__ constexpr int g_off(int r, int c) { return k_off<64>(r, c); }

__device__ __forceinline__ void tile_of(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nt = tiles_m * tiles_n;
  const int xcd = id & 7, slot = id >> 3;
  const int q = nt >> 3, rmd = nt & 7;
  const int t = (xcd < rmd ? xcd * (q + 1) : rmd * (q + 1) + (xcd - rmd) * q) + slot;
  const int per_group = GROUP_M * tiles_n;
  const int g = t / per_group, first = g * GROUP_M;
  const int gsize = min(GROUP_M, tiles_m - first);
  const int w = t - g * per_group;
  tm = first + w % gsize;
  tn = w / gsize;
}

// Byte offset of A row m (all K blocks of the row share it; the block's own
// offset goes in the scalar offset), or kOob past the last row.
template <int MODE>
__device__ __forceinline__ unsigned a_row_off(const ProjArgs& a, int m) {
  if (m >= a.M) return kOob;
  if constexpr (MODE == PROJ_OUT) {
    // row (b, t) of out.transpose(1, 2).reshape(B, T, H*hd): head h's hd values
    // sit at o[b, h, t, :]; the row part is b*H*T*hd + t*hd (elements)
    const int b = m / a.T, t = m - b * a.T;
    return (unsigned)(((long)b * a.H * a.T + t) * a.hd * 2);
  } else {
    return (unsigned)((long)m * a.K * 2);
  }
}
// Byte offset of K block kb within a row (added as the scalar offset).
template <int MODE>
__device__ __forceinline__ unsigned a_k_off(const ProjArgs& a, int kb) {
  const int k0 = kb * GBK;
  if constexpr (MODE == PROJ_OUT) {
    const int h = k0 / a.hd, d0 = k0 - h * a.hd;  // a 64-wide block never straddles heads (hd % 64 == 0)
    return (unsigned)(((long)h * a.T * a.hd + d0) * 2);
  } else {
    return (unsigned)(k0 * 2);
  }
}

__device__ __forceinline__ void store_bf16(void* base, long idx, float v) {
  reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16_bits(v);
}

template <int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void proj_gemm_kernel(ProjArgs a) {
  // two stages of [A slice | W slice]
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * GTILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_m = (a.M + GBM - 1) / GBM, tiles_n = (a.N + GBN - 1) / GBN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * GBM, n0 = tn * GBN;

  // LDS-DMA: this wave's instruction i of an operand slice fills LDS bytes
  // 1024 (wave*GPW + i) + 16 lane, i.e. row r = 8 (wave*GPW + i) + lane/8 at
  // physical chunk lane%8, which holds logical chunk (lane%8) ^ swz(r).
  unsigned aoff[GPW], woff[GPW];
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    const int r = 8 * (wave * GPW + i) + (lane >> 3);
    const int lc = (lane & 7) ^ ((r >> 1) & 7);
    const unsigned ar = a_row_off<MODE>(a, m0 + r);
    aoff[i] = ar == kOob ? kOob : ar + lc * 16;
    woff[i] = n0 + r < a.N ? (unsigned)((long)(n0 + r) * a.K * 2) + lc * 16 : kOob;
  }
  static_assert(g_off(9, 3) == 9 * 128 + ((3 ^ 4) << 4), "the DMA swizzle above is k_off<64>'s");
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.a, (int)a.a_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, (int)a.w_bytes);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(a.a, 0);  // empty: reads nothing, writes zeros
  // Instructions 2s, 2s+1 of each operand slice of block kb (of GPW = 8 per
  // wave), so a block's DMA goes out in four parts between its MFMAs. Past the
  // last block the descriptors are empty: the loads read no memory and write
  // zeros into the stage the finished block before it used.
  auto issue_part = [&](int kb, unsigned char* sa, unsigned char* sw, int part) __attribute__((always_inline)) {
    const bool live = kb < a.K / GBK;
    const unsigned ka = live ? a_k_off<MODE>(a, kb) : 0u, kw = live ? (unsigned)(kb * GBK * 2) : 0u;
    const __amdgpu_buffer_rsrc_t qa = live ? ra : rz, qw = live ? rw : rz;
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int i = 2 * part; i < 2 * part + 2; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qa, (LDS void*)(sa + 1024 * (wave * GPW + i)), 16, aoff[i], ka, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qw, (LDS void*)(sw + 1024 * (wave * GPW + i)), 16, woff[i], kw, 0, 0);
    }
#endif
  };
  auto issue = [&](int kb, unsigned char* sa, unsigned char* sw) __attribute__((always_inline)) {
#pragma unroll
    for (int part = 0; part < GPW / 2; ++part) issue_part(kb, sa, sw, part);
  };
  static_assert(GPW == 2 * (GBK / 16), "two instructions per operand slice per 16-deep step");

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int n = lane & 31, hf = lane >> 5;
  // one 64-wide K block: 4 steps of 16, each 4 A and 4 W operand reads and 16
  // MFMAs. Fenced order per step: the operand reads of step s+1, then the 16
  // MFMAs of step s (whose operands were requested a whole step earlier) with
  // one LDS-DMA instruction of the next block after every four of them, so the
  // DMA issue never holds the matrix core up in a burst.
  auto multiply = [&](const unsigned char* sa, const unsigned char* sw, unsigned char* na, unsigned char* nw,
                      int kn) __attribute__((always_inline)) {
    LdsBytes la = (LdsBytes)sa, lw = (LdsBytes)sw;
    bf16x8 av[2][4], wv[2][4];
    auto load = [&](int s, int set) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        av[set][i] = *reinterpret_cast<const LDS bf16x8*>(la + g_off(wm * 128 + 32 * i + n, 2 * s + hf));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wv[set][j] = *reinterpret_cast<const LDS bf16x8*>(lw + g_off(wn * 128 + 32 * j + n, 2 * s + hf));
    };
    load(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < GBK / 16; ++s) {
      if (s + 1 < GBK / 16) load(s + 1, (s + 1) & 1);
      issue_part(kn, na, nw, s);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[s & 1][i], wv[s & 1][j], acc[i][j], 0, 0, 0);
      if (s + 1 < GBK / 16) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nk = a.K / GBK;
  issue(0, smem, smem + GTILE);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // Step: multiply block kb while its DMA parts bring block kb+1 into the
  // other stage (released by the barrier that ended the previous step), wait
  // for this wave's DMA and meet the others (block kb+1 is then complete and
  // block kb's stage free).
  for (int kb = 0; kb < nk; ++kb) {
    unsigned char* cur = smem + (kb & 1) * 2 * GTILE;
    unsigned char* nxt = smem + ((kb + 1) & 1) * 2 * GTILE;
    multiply(cur, cur + GTILE, nxt, nxt + GTILE, kb + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue, one 32-row block of the wave's quarter at a time, through
  // LDS (free after the last barrier): the lanes write the accumulators of
  // block row i ([32 rows][128 columns] fp32, rows padded to EPS floats), then
  // read them back as 4 rows x 16 column groups of 8 per pass, so that each
  // lane rotates 4 whole pairs and stores 16 contiguous bytes.
  constexpr int EPS = 132;
  float* ep = reinterpret_cast<float*>(smem) + wave * 32 * EPS;
  const int cg = lane & 15;                    // column group: columns 8cg .. 8cg+7 of the quarter
  const int col0 = n0 + wn * 128 + 8 * cg;     // its first global column
  const bool col_ok = col0 < a.N;              // N is a multiple of 8: a group is in or out
  int sec = 0, head = 0, d0 = 0, heads = 1;
  bool rot = false;
  double rev[4] = {0.0, 0.0, 0.0, 0.0};
  if constexpr (MODE != PROJ_OUT) {
    // 8 columns lie inside one head of one section (hd % 8 == 0)
    const int Hhd = a.H * a.hd, KVhd = a.KV * a.hd;
    sec = col0 < Hhd ? 0 : (col0 < Hhd + KVhd ? 1 : 2);
    const int cs = col0 - (sec == 0 ? 0 : (sec == 1 ? Hhd : Hhd + KVhd));
    head = cs / a.hd;
    d0 = cs - head * a.hd;
    heads = sec == 0 ? a.H : a.KV;
    rot = a.rope && sec < 2 && col_ok;
    if (rot) {
#pragma unroll
      for (int u = 0; u < 4; ++u) rev[u] = a.freqs.rev[(d0 >> 1) + u];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) ep[(8 * (r >> 2) + 4 * hf + (r & 3)) * EPS + 32 * j + n] = acc[i][j][r];
    // (LDS operations of one wave complete in order: the reads below see these writes)
    for (int pass = 0; pass < 8; ++pass) {
      const int row = 4 * pass + (lane >> 4);
      const int m = m0 + wm * 128 + 32 * i + row;
      const float4 lo = *reinterpret_cast<const float4*>(ep + row * EPS + 8 * cg);
      const float4 hi = *reinterpret_cast<const float4*>(ep + row * EPS + 8 * cg + 4);
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      if (m >= a.M || !col_ok) continue;
      const int b = m / a.T, t = m - b * a.T;
      if constexpr (MODE == PROJ_OUT) {
        const long idx = (long)m * a.N + col0;
        if (a.out_bf16) {
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.y) + idx) =
              make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
        } else {
          float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + idx);
          dst[0] = lo;
          dst[1] = hi;
        }
      } else {
        int pos;
        bool ok = true;
        if constexpr (MODE == PROJ_QKV_CACHE) {
          const int L = a.lens[b];
          ok = L >= 0 && L <= a.Lmax - a.T;
          pos = L + t;
        } else {
          pos = a.pos0 + t;
        }
        if (rot) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float c, sn;
            rope_cos_sin(pos, rev[u], c, sn);
            const float x0 = v[2 * u], x1 = v[2 * u + 1];
            v[2 * u] = rot0(x0, x1, c, sn);
            v[2 * u + 1] = rot1(x0, x1, c, sn);
          }
        }
        const uint4 pk = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                    pack_bf16x2(v[6], v[7]));
        if (sec == 0) {
          const long qi = (((long)b * heads + head) * a.T + t) * a.hd + d0;
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.q) + qi) =
              ok ? pk : make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);  // bf16 NaN
        } else if (ok) {
          long di;
          void* base;
          if constexpr (MODE == PROJ_QKV_CACHE) {
            di = (((long)b * heads + head) * a.Lmax + pos) * a.hd + d0;
            base = sec == 1 ? a.k_cache : a.v_cache;
          } else {
            di = (((long)b * heads + head) * a.T + t) * a.hd + d0;
            base = sec == 1 ? a.k : a.v;
          }
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(base) + di) = pk;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_proj(const ProjArgs& a, int mode, hipStream_t s, const TimingHook& tm) {
  const int tiles = ((a.M + GBM - 1) / GBM) * ((a.N + GBN - 1) / GBN);
  hipError_t e;
  if ((e = tm.before(s)) != hipSuccess) return e;
  if (mode == PROJ_QKV) {
    hipLaunchKernelGGL(proj_gemm_kernel<PROJ_QKV>, dim3(tiles), dim3(256), 0, s, a);
  } else if (mode == PROJ_QKV_CACHE) {
    hipLaunchKernelGGL(proj_gemm_kernel<PROJ_QKV_CACHE>, dim3(tiles), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(proj_gemm_kernel<PROJ_OUT>, dim3(tiles), dim3(256), 0, s, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return tm.after(s);
}

}  // namespace attn
