// KV-cache decode: cache append, split-KV partial attention, log-sum-exp merge.
//
// The new token of sequence b sits at position L = lens[b]. Its key is rotated
// at L and written with its value at cache slot L (a cache pre-allocated and
// written by position, as the roadmap of "Building Grouped-Query Attention with
// RoPE and Flash Attention from Scratch" describes); its query, rotated at L,
// attends slots 0..L. Keys are cut into splits of kDecodeSplit slots; each split
// yields an unnormalised partial output with its running max m and denominator
// l, and the merge combines them with weights 2^(m_s - M): the same rescaling
// rule as the online-softmax recurrences of "Building a Transformer from
// Scratch", Part 3, applied across splits instead of along one loop.
#include "attn_internal.h"

namespace attn {

namespace {

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.4426950408889634f;

template <int BF16>
__device__ __forceinline__ float ld(const void* base, long i) {
  if constexpr (BF16) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
  } else {
    return reinterpret_cast<const float*>(base)[i];
  }
}

__device__ __forceinline__ bool bad_len(int L, int Lmax) { return L < 0 || L >= Lmax; }

// Grid (KV, B), hd/2 threads (one interleaved pair each): rotate k_new at L and
// write slot L of both caches (vector-ALU path; the MFMA split kernel does this
// itself).
template <int BF16>
__global__ void decode_append_kernel(DecodeArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, p = threadIdx.x;
  const int L = a.lens[b];
  if (bad_len(L, a.Lmax) || 2 * p >= a.hd) return;
  float c = 1.f, s = 0.f;
  if (a.rope) rope_cos_sin(L, a.freqs.rev[p], c, s);
  const long src = ((long)b * a.KV + g) * a.hd + 2 * p;
  const long dst = (((long)b * a.KV + g) * a.Lmax + L) * a.hd + 2 * p;
  const float x0 = ld<BF16>(a.k_new, src), x1 = ld<BF16>(a.k_new, src + 1);
  const float y0 = rot0(x0, x1, c, s), y1 = rot1(x0, x1, c, s);
  if constexpr (BF16) {
    reinterpret_cast<uint32_t*>(a.k_cache)[dst >> 1] = pack_bf16x2(y0, y1);
    reinterpret_cast<uint32_t*>(a.v_cache)[dst >> 1] = reinterpret_cast<const uint32_t*>(a.v_new)[src >> 1];
  } else {
    reinterpret_cast<float2*>(a.k_cache)[dst >> 1] = make_float2(y0, y1);
    reinterpret_cast<float2*>(a.v_cache)[dst >> 1] = reinterpret_cast<const float2*>(a.v_new)[src >> 1];
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Vector-ALU split kernel. Grid (nsplit, H, B), 256 threads: thread = key slot
// for the scores, thread = head-dim index for the partial output.
template <int BF16, int HD>
__global__ __launch_bounds__(256) void decode_split_valu_kernel(DecodeArgs a) {
  constexpr int C = kDecodeSplit;
  static_assert(C == 256, "one key per thread");
  const int sp = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = a.lens[b];
  if (bad_len(L, a.Lmax)) return;
  const int k0 = sp * C;
  if (k0 > L) return;
  const int k1 = min(L + 1, k0 + C);
  const int g = h / a.group;
  const int t = threadIdx.x;
  __shared__ float qs[HD];
  __shared__ float ps[C];
  __shared__ float red[4];

  if (t < HD / 2) {
    const long qi = ((long)b * a.H + h) * HD + 2 * t;
    float x0 = ld<BF16>(a.q, qi), x1 = ld<BF16>(a.q, qi + 1);
    if (a.rope) {
      float c, s;
      rope_cos_sin(L, a.freqs.rev[t], c, s);
      const float y0 = rot0(x0, x1, c, s), y1 = rot1(x0, x1, c, s);
      x0 = y0;
      x1 = y1;
    }
    qs[2 * t] = x0 * a.scale_log2;
    qs[2 * t + 1] = x1 * a.scale_log2;
  }
  __syncthreads();
  const long cbase = ((long)b * a.KV + g) * (long)a.Lmax * HD;
  const float slope2 = a.alibi ? alibi_slope(a.alibi, h, a.H) * kLog2e : 0.f;
  const int key = k0 + t;
  float x = -INFINITY;
  if (key < k1) {
    float dot = 0.f;
    for (int d = 0; d < HD; ++d) dot = fmaf(qs[d], ld<BF16>(a.k_cache, cbase + (long)key * HD + d), dot);
    x = dot - slope2 * (float)(L - key);
  }
  const int w = t >> 6, lane = t & 63;
  float mx = wave_max(x);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float p = (key < k1) ? exp2f(x - mx) : 0.f;
  ps[t] = p;
  __syncthreads();
  float sm = wave_sum(p);
  __syncthreads();
  if (lane == 0) red[w] = sm;
  __syncthreads();
  sm = red[0] + red[1] + red[2] + red[3];
  const long pidx = ((long)b * a.H + h) * a.nsplit + sp;
  if (t < HD) {
    float o = 0.f;
    for (int j = 0; j < k1 - k0; ++j) o = fmaf(ps[j], ld<BF16>(a.v_cache, cbase + (long)(k0 + j) * HD + t), o);
    a.part_o[pidx * HD + t] = o;
  }
  if (t == 0) a.part_ml[pidx] = make_float2(mx, sm);
}

// ---------------------------------------------------------------- MFMA split kernel
// bf16, hd in {64, 128}, group = H/KV <= 16. Grid (KV*B, nsplit), 4 waves,
// kSplitMfma (or kSplitMfmaLong) key slots per workgroup.
// The group's query heads are the columns of S^T = K Q^T computed with
// v_mfma_f32_16x16x32_bf16, so each K/V byte is read from memory once for all of
// them. Each wave streams 32-key tiles (interleaved with the other waves) through
// a private LDS region, with the next tile's global loads in flight while the
// current one is computed (no workgroup barrier inside the loop). K is stored
// row-major with an XOR swizzle and read as the A operand; V is stored row-major
// with an XOR swizzle and read as V^T with ds_read_b64_tr_b16, the transposing
// LDS load of gfx950. Key rows are permuted so that a lane's accumulator
// registers hold 8 consecutive keys, which feed O^T = V^T P^T as its B operand
// straight from registers. Each workgroup rotates the query with a cos/sin table
// for position L in LDS; the workgroup whose split holds slot L also appends the
// new key/value (cache write plus an LDS patch of its own tile). The four waves'
// (m, l, O) are merged in LDS and one partial per head is written.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;  // keys per wave tile
constexpr int kWaves = 4;

// MFMA row rho (0..15) of key block kb (0 or 1) holds tile key 8*(rho/4) + 4*kb + rho%4.
__device__ __forceinline__ int kperm16(int rho, int kb) { return ((rho >> 2) << 3) | (kb << 2) | (rho & 3); }

template <int HD>
__device__ __forceinline__ int dk_off(int r, int c) {  // K tile: 16-byte chunk c of key row r
  if constexpr (HD == 128) {
    return r * 256 + ((c ^ ((r & 3) | ((r >> 3) << 2))) << 4);
  } else {
    return r * 128 + ((c ^ (((r >> 1) & 1) | ((r >> 3) << 1))) << 4);
  }
}
template <int HD>
__device__ __forceinline__ int dv_off(int r, int c) {  // V tile: 16-byte chunk c of key row r
  if constexpr (HD == 128) {
    return r * 256 + ((c ^ (((r & 3) << 1) | (((r >> 3) & 1) << 3))) << 4);
  } else {
    return r * 128 + ((c ^ ((((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2))) << 4);
  }
}

// fp8 cache: OCP E4M3 code of x (x already divided by the scale): |x| clamped
// to 448 and rounded to nearest, ties to even mantissa; subnormals below 2^-6
// are multiples of 2^-9; the sign bit is x's.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sgn = (bits >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.f);
  if (a < 0.015625f) return sgn | (uint32_t)rintf(a * 512.f);  // 0..8 (8 is the smallest normal)
  const uint32_t ab = __float_as_uint(a);
  int e = (int)(ab >> 23) - 127;
  uint32_t m = (ab >> 20) & 7u;
  const uint32_t rem = ab & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
  if (m == 8u) {
    m = 0u;
    ++e;
  }
  return sgn | ((uint32_t)(e + 7) << 3) | m;
}

// Four E4M3 codes (one 32-bit word) -> four bf16 (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t w) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

template <int HD, int TPW, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_split_mfma_kernel(DecodeArgs a) {
  constexpr int SPLIT = kWaves * kTile * TPW;  // key slots per workgroup
  constexpr int KCH = HD / 8;                 // 16-byte bf16 chunks per row (in LDS)
  constexpr int EB = FP8 ? 1 : 2;             // cache bytes per element
  constexpr int GCH = HD * EB / 16;           // 16-byte chunks per cache row (in memory)
  constexpr int TILE_BYTES = kTile * HD * 2;  // one K or V tile in LDS (bf16)
  constexpr int LOADS = kTile * GCH / 64;     // 16-byte loads per lane per tensor
  constexpr int NSLOT = FP8 ? 4 : 2;          // tiles in flight per wave (about the same bytes either way)
  __shared__ __attribute__((aligned(16))) unsigned char smem[kWaves * 2 * TILE_BYTES];
  __shared__ float mer_m[kWaves][16];
  __shared__ float mer_l[kWaves][16];

  // Grid (KV*B, nsplit): every sequence's first split is dispatched before any
  // second split, so the blocks past a short sequence's end (which exit at once)
  // cluster at the end of the dispatch order.
  const int sp = blockIdx.y, kvh = blockIdx.x % a.KV, b = blockIdx.x / a.KV;
  const int L = a.lens[b];
  if (bad_len(L, a.Lmax)) return;
  const int nk = L + 1;
  const int k0 = sp * SPLIT;
  if (k0 >= nk) return;
  // the wave index read from lane 0, so the compiler knows it is wave-uniform:
  // the buffer descriptors built from it stay scalar (no per-load waterfall loop)
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n = lane & 15, g = lane >> 4;
  const int G = a.group;
  const bool qcol = n < G;
  const int head = kvh * G + (qcol ? n : 0);

  const long cbase = ((long)b * a.KV + kvh) * (long)a.Lmax * HD;  // elements
  const unsigned char* Kg = reinterpret_cast<const unsigned char*>(a.k_cache) + cbase * EB;
  const unsigned char* Vg = reinterpret_cast<const unsigned char*>(a.v_cache) + cbase * EB;
  unsigned char* kl = smem + wave * 2 * TILE_BYTES;
  unsigned char* vl = kl + TILE_BYTES;

  // NSLOT tiles of K/V in flight per wave: slot t % NSLOT holds tile t until it
  // is written to LDS, then receives tile t + NSLOT. The first ones go out
  // before the rotary table and the query set-up, which then hide under their
  // latency.
  // Buffer descriptors start at the tile and end at key slot nk or at the
  // tile's end, whichever comes first, so rows past the sequence end read as
  // zero and the 32-bit descriptor size never exceeds one tile, however long
  // the cache. (The wave whose tile covers slot L may read it before the new
  // key lands there; it patches that row in LDS.)
  uint4 kr[NSLOT][LOADS], vr[NSLOT][LOADS];
  // Issued unconditionally (a tile at or past the sequence end gets an empty
  // descriptor: every lane reads zero and no memory is touched), so the wait
  // before each tile's LDS write counts only that tile's loads; a conditional
  // issue would make the compiler drain every load in flight there.
  auto load_tile = [&](int slot, int ts) {
    const int bytes = min(max(nk - ts, 0), kTile) * HD * EB;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg + (long)ts * HD * EB, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg + (long)ts * HD * EB, bytes);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      kr[slot][i] = buffer_load16_stream(rk, 16 * (lane + 64 * i));
      vr[slot][i] = buffer_load16_stream(rv, 16 * (lane + 64 * i));
    }
  };
  const auto tile_start = [&](int t) { return k0 + (t * kWaves + wave) * kTile; };
#pragma unroll
  for (int t = 0; t < NSLOT; ++t)
    if (t < TPW) load_tile(t, tile_start(t));

  // cos/sin of the rotary angle at position L for every pair, shared in LDS.
  __shared__ float2 cs_tab[HD / 2];
  if (tid < HD / 2) {
    float c = 1.f, sn = 0.f;
    if (a.rope) rope_cos_sin(L, a.freqs.rev[tid], c, sn);
    cs_tab[tid] = make_float2(c, sn);
  }
  // This split holds the new token's slot L: its workgroup writes the rotated
  // key and the value to the cache, and the wave whose tile covers slot L
  // patches that row of its LDS tile (it never reads slot L back from memory).
  const bool own_slot = a.append && L >= k0 && L < k0 + SPLIT;
  uint32_t knew = 0, vnew = 0;  // lane p < HD/2: pair p of R(L) k_new and v_new (bf16x2, as read back)
  const long cslot = (((long)b * a.KV + kvh) * a.Lmax + L) * HD;
  const long nslot = ((long)b * a.KV + kvh) * HD;
  __syncthreads();
  if (own_slot && lane < HD / 2) {
    const uint32_t kw = reinterpret_cast<const uint32_t*>(a.k_new)[(nslot >> 1) + lane];
    const uint32_t vw = reinterpret_cast<const uint32_t*>(a.v_new)[(nslot >> 1) + lane];
    const float2 t = cs_tab[lane];
    const float x0 = bf16_bits_to_f32(kw & 0xffffu), x1 = bf16_bits_to_f32(kw >> 16);
    const float y0 = rot0(x0, x1, t.x, t.y), y1 = rot1(x0, x1, t.x, t.y);
    if constexpr (FP8) {
      // stored as E4M3 codes of value / scale; the LDS patch holds what a read returns
      const uint32_t kc = e4m3_code(y0 / a.k_scale) | (e4m3_code(y1 / a.k_scale) << 8);
      const uint32_t vc = e4m3_code(bf16_bits_to_f32(vw & 0xffffu) / a.v_scale) |
                          (e4m3_code(bf16_bits_to_f32(vw >> 16) / a.v_scale) << 8);
      knew = e4m3x4_to_bf16(kc).x;
      vnew = e4m3x4_to_bf16(vc).x;
      if (wave == 0) {
        reinterpret_cast<uint16_t*>(a.k_cache)[(cslot >> 1) + lane] = (uint16_t)kc;
        reinterpret_cast<uint16_t*>(a.v_cache)[(cslot >> 1) + lane] = (uint16_t)vc;
      }
    } else {
      knew = pack_bf16x2(y0, y1);
      vnew = vw;
      if (wave == 0) {
        reinterpret_cast<uint32_t*>(a.k_cache)[(cslot >> 1) + lane] = knew;
        reinterpret_cast<uint32_t*>(a.v_cache)[(cslot >> 1) + lane] = vnew;
      }
    }
  }

  // Q^T B operand: column n = head kvh*G + n rotated at L (zeros for n >= G);
  // k-step s holds dims 32s + 8g .. +7, i.e. pairs 16s + 4g .. +3.
  bf16x8_t qf[HD / 32];
  {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                                      ((long)b * a.H + head) * HD);
#pragma unroll
    for (int s = 0; s < HD / 32; ++s) {
      const uint4 wv = qcol ? src[4 * s + g] : make_uint4(0, 0, 0, 0);
      const uint32_t w4[4] = {wv.x, wv.y, wv.z, wv.w};
      uint32_t d[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float2 t = cs_tab[16 * s + 4 * g + p];
        const float x0 = bf16_bits_to_f32(w4[p] & 0xffffu), x1 = bf16_bits_to_f32(w4[p] >> 16);
        d[p] = pack_bf16x2(rot0(x0, x1, t.x, t.y), rot1(x0, x1, t.x, t.y));
      }
      qf[s] = __builtin_bit_cast(bf16x8_t, make_uint4(d[0], d[1], d[2], d[3]));
    }
  }
  const float c2 = FP8 ? a.scale_log2 * a.k_scale : a.scale_log2;  // K's scale folds into the scores
  const float slope2 = a.alibi ? alibi_slope(a.alibi, head, a.H) * kLog2e : 0.f;

  f32x4_t oacc[HD / 16];
#pragma unroll
  for (int db = 0; db < HD / 16; ++db) oacc[db] = f32x4_t{};
  float m_run = -INFINITY, l_run = 0.f;

#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int ts = tile_start(t);
    if (ts >= nk) break;
    const int slot = t % NSLOT;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int e = lane + 64 * i;
      const int r = e / GCH, c = e % GCH;
      if constexpr (FP8) {  // 16 codes -> two bf16 chunks 2c, 2c+1 of the row
        const uint4 kq = kr[slot][i], vq = vr[slot][i];
        const uint2 k0 = e4m3x4_to_bf16(kq.x), k1 = e4m3x4_to_bf16(kq.y), k2 = e4m3x4_to_bf16(kq.z),
                    k3 = e4m3x4_to_bf16(kq.w);
        const uint2 v0 = e4m3x4_to_bf16(vq.x), v1 = e4m3x4_to_bf16(vq.y), v2 = e4m3x4_to_bf16(vq.z),
                    v3 = e4m3x4_to_bf16(vq.w);
        *reinterpret_cast<uint4*>(kl + dk_off<HD>(r, 2 * c)) = make_uint4(k0.x, k0.y, k1.x, k1.y);
        *reinterpret_cast<uint4*>(kl + dk_off<HD>(r, 2 * c + 1)) = make_uint4(k2.x, k2.y, k3.x, k3.y);
        *reinterpret_cast<uint4*>(vl + dv_off<HD>(r, 2 * c)) = make_uint4(v0.x, v0.y, v1.x, v1.y);
        *reinterpret_cast<uint4*>(vl + dv_off<HD>(r, 2 * c + 1)) = make_uint4(v2.x, v2.y, v3.x, v3.y);
      } else {
        *reinterpret_cast<uint4*>(kl + dk_off<HD>(r, c)) = kr[slot][i];
        *reinterpret_cast<uint4*>(vl + dv_off<HD>(r, c)) = vr[slot][i];
      }
    }
    if (own_slot && L >= ts && L < ts + kTile && lane < HD / 2) {
      const int r = L - ts;  // pair `lane` sits in chunk lane/4, bytes 4*(lane%4)
      *reinterpret_cast<uint32_t*>(kl + dk_off<HD>(r, lane >> 2) + 4 * (lane & 3)) = knew;
      *reinterpret_cast<uint32_t*>(vl + dv_off<HD>(r, lane >> 2) + 4 * (lane & 3)) = vnew;
    }
    if (t + NSLOT < TPW) load_tile(slot, tile_start(t + NSLOT));

    // S^T = K Q^T for the tile's two 16-key blocks
    f32x4_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4_t{};
      const int row = kperm16(n, kb);
#pragma unroll
      for (int s = 0; s < HD / 32; ++s) {
        const uint4 av = *reinterpret_cast<const uint4*>(kl + dk_off<HD>(row, 4 * s + g));
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), qf[s], sacc[kb], 0, 0, 0);
      }
    }
    // tv[4*kb + r] is key ts + 8g + 4kb + r
    float tv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = ts + 8 * g + i;
      float x = sacc[i >> 2][i & 3] * c2;
      if (a.alibi) x = fmaf(slope2, (float)(key - L), x);
      x = key < nk ? x : -INFINITY;
      tv[i] = x;
      mx = fmaxf(mx, x);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      tv[i] = __builtin_amdgcn_exp2f(tv[i] - m_new);
      lsum += tv[i];
    }
    l_run = fmaf(l_run, alpha, lsum);
    m_run = m_new;
    const bf16x8_t pb = __builtin_bit_cast(
        bf16x8_t, make_uint4(pack_bf16x2(tv[0], tv[1]), pack_bf16x2(tv[2], tv[3]), pack_bf16x2(tv[4], tv[5]),
                             pack_bf16x2(tv[6], tv[7])));
    // O^T += V^T P^T. Transposing load: source lane i of 16-lane group g points at
    // row 8g + i/4 (+4), columns d0 + 4*(i%4); lane i receives V[rows][d0 + i].
    const int li = lane & 15;
#pragma unroll
    for (int db = 0; db < HD / 16; ++db) {
      oacc[db] *= alpha;
      const int col = 16 * db + 4 * (li & 3);
      const int r = 8 * g + (li >> 2);
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(vl + dv_off<HD>(r, col >> 3) + (col & 7) * 2));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(vl + dv_off<HD>(r + 4, col >> 3) + (col & 7) * 2));
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, oacc[db], 0, 0, 0);
    }
  }

  // ---- merge the four waves: per column n, M = max_w m_w, weights 2^(m_w - M)
  float l_col = l_run + __shfl_xor(l_run, 16);
  l_col += __shfl_xor(l_col, 32);
  if (g == 0) {
    mer_m[wave][n] = m_run;
    mer_l[wave][n] = l_col;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mer_m[w][n]);
  const float wgt = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
  float* ob = reinterpret_cast<float*>(smem);  // [wave][16][HD], reuses the tile space
  if (qcol) {
#pragma unroll
    for (int db = 0; db < HD / 16; ++db) {
      const int d = 16 * db + 4 * g;
      *reinterpret_cast<float4*>(ob + (wave * 16 + n) * HD + d) =
          make_float4(oacc[db][0] * wgt, oacc[db][1] * wgt, oacc[db][2] * wgt, oacc[db][3] * wgt);
    }
  }
  __syncthreads();
  for (int e = tid; e < G * HD; e += 256) {
    const int col = e / HD, d = e % HD;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) o += ob[(w * 16 + col) * HD + d];
    const long pidx = ((long)b * a.H + kvh * G + col) * a.nsplit + sp;
    a.part_o[pidx * HD + d] = FP8 ? o * a.v_scale : o;  // V's scale, applied once per partial
    if (d == 0) {
      float Mc = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) Mc = fmaxf(Mc, mer_m[w][col]);
      float lt = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = mer_m[w][col];
        lt += (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - Mc) * mer_l[w][col];
      }
      a.part_ml[pidx] = make_float2(Mc, lt);
    }
  }
}

// Merge the partials of one (b, h): one wave, lanes in parallel over splits for
// the max and the weights, then each lane accumulates two head-dim entries over
// the splits (independent loads). Grid (H, B), 64 threads.
template <int HD>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int L = a.lens[b];
  const long orow = ((long)b * a.H + h) * HD;
  float res[2] = {0.f, 0.f};
  float lse;
  if (bad_len(L, a.Lmax)) {
    res[0] = res[1] = __builtin_nanf("");
    lse = res[0];
  } else {
    const int ns = (L + 1 + a.split - 1) / a.split;
    const long p0 = ((long)b * a.H + h) * a.nsplit;
    float M = -INFINITY;
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, a.part_ml[p0 + s].x);
    M = wave_max(M);
    float den = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 64) {
      float w = 0.f;
      if (s0 + lane < ns) {
        const float2 ml = a.part_ml[p0 + s0 + lane];
        w = exp2f(ml.x - M);
        den = fmaf(w, ml.y, den);
      }
      const int cnt = min(64, ns - s0);
      // 8 splits per step with all loads issued before the multiply-adds
      for (int j0 = 0; j0 < cnt; j0 += 8) {
        float v[8][2];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int d = lane + 64 * k;
            v[u][k] = (j0 + u < cnt && d < HD) ? a.part_o[(p0 + s0 + j0 + u) * HD + d] : 0.f;
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wj = __shfl(w, j0 + u);
          res[0] = fmaf(wj, v[u][0], res[0]);
          res[1] = fmaf(wj, v[u][1], res[1]);
        }
      }
    }
    den = wave_sum(den);
    res[0] /= den;
    res[1] /= den;
    lse = (M + log2f(den)) * kLn2;
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int d = lane + 64 * k;
    if (d >= HD) break;
    if (a.out_bf16) {
      reinterpret_cast<uint16_t*>(a.out)[orow + d] = f32_to_bf16_bits(res[k]);
    } else {
      reinterpret_cast<float*>(a.out)[orow + d] = res[k];
    }
  }
  if (a.lse && lane == 0) a.lse[(long)b * a.H + h] = lse;
}

}  // namespace

bool decode_mfma_supported(const DecodeArgs& a, int bf16) {
  return bf16 && (a.hd == 64 || a.hd == 128) && a.group <= 16;
}

int decode_split_for(const DecodeArgs& a, int bf16) {
  if (!decode_mfma_supported(a, bf16)) return kDecodeSplit;
  // MFMA path: the longer split when it still gives at least four workgroups
  // per CU (measured on the 64-sequence, 8-KV-head cache: 5.6 -> 6.0 TB/s), so
  // the per-workgroup set-up is amortised over more keys.
  const bool long_split = (long)a.KV * a.B * ((a.Lmax + kSplitMfmaLong - 1) / kSplitMfmaLong) >= 1024;
  // fp8: half the bytes per key, so twice the keys per workgroup for the same set-up cost
  const bool fp8_split = a.fp8 && (long)a.KV * a.B * ((a.Lmax + kSplitMfmaFp8 - 1) / kSplitMfmaFp8) >= 1024;
  return fp8_split ? kSplitMfmaFp8 : (long_split ? kSplitMfmaLong : kSplitMfma);
}

namespace {

template <int BF16, int HD>
hipError_t launch_decode_hd(const DecodeArgs& a0, hipStream_t s, const TimingHook& tm) {
  DecodeArgs a = a0;
  const bool mfma = decode_mfma_supported(a, BF16);
  if (a.fp8 && !mfma) return hipErrorInvalidValue;  // the host checks this first
  a.split = decode_split_for(a, BF16);
  a.nsplit = (a.Lmax + a.split - 1) / a.split;
  hipError_t e = hipSuccess;
  if (!mfma && a.append) {  // the MFMA split kernel appends the new token itself
    hipLaunchKernelGGL(decode_append_kernel<BF16>, dim3(a.KV, a.B), dim3(HD / 2), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = tm.before(s)) != hipSuccess) return e;
  if (mfma) {
    if constexpr (HD == 64 || HD == 128) {
      constexpr int TPW = kSplitMfma / (kWaves * kTile);
      const dim3 grid(a.KV * a.B, a.nsplit);
      if (a.fp8) {
        if (a.split == kSplitMfmaFp8) {
          hipLaunchKernelGGL((decode_split_mfma_kernel<HD, 4 * TPW, true>), grid, dim3(256), 0, s, a);
        } else if (a.split == kSplitMfmaLong) {
          hipLaunchKernelGGL((decode_split_mfma_kernel<HD, 2 * TPW, true>), grid, dim3(256), 0, s, a);
        } else {
          hipLaunchKernelGGL((decode_split_mfma_kernel<HD, TPW, true>), grid, dim3(256), 0, s, a);
        }
      } else if (a.split == kSplitMfmaLong) {
        hipLaunchKernelGGL((decode_split_mfma_kernel<HD, 2 * TPW, false>), grid, dim3(256), 0, s, a);
      } else {
        hipLaunchKernelGGL((decode_split_mfma_kernel<HD, TPW, false>), grid, dim3(256), 0, s, a);
      }
    }
  } else {
    hipLaunchKernelGGL((decode_split_valu_kernel<BF16, HD>), dim3(a.nsplit, a.H, a.B), dim3(256), 0, s, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = tm.after(s)) != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<HD>), dim3(a.H, a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int BF16>
hipError_t launch_decode_dt(const DecodeArgs& a, hipStream_t s, const TimingHook& tm) {
  switch (a.hd) {
    case 8: return launch_decode_hd<BF16, 8>(a, s, tm);
    case 16: return launch_decode_hd<BF16, 16>(a, s, tm);
    case 32: return launch_decode_hd<BF16, 32>(a, s, tm);
    case 64: return launch_decode_hd<BF16, 64>(a, s, tm);
    case 128: return launch_decode_hd<BF16, 128>(a, s, tm);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int bf16, hipStream_t s, const TimingHook& tm) {
  return bf16 ? launch_decode_dt<1>(a, s, tm) : launch_decode_dt<0>(a, s, tm);
}

}  // namespace attn
