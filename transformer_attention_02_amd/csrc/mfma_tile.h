// Tile machinery shared by the matrix-core attention kernels (forward and
// backward): operand types, the 64-key tile layout in LDS, its XOR swizzles,
// the row permutation that lines accumulator registers up with the next
// contraction's operand, and direct global -> LDS staging of K/V tiles.
#pragma once

#include "attn_internal.h"

namespace attn {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 64;  // keys per tile

template <int HD>
struct Cfg {
  static constexpr int KCH = HD / 8;               // 16-byte chunks per key row
  static constexpr int K_BYTES = BN * HD * 2;      // K tile, row-major [key][hd], XOR-swizzled chunks
  static constexpr int V_BYTES = BN * HD * 2;      // V tile, row-major [key][hd], XOR-swizzled chunks
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int DMA = K_BYTES / 1024;       // 1 KiB LDS-DMA wave instructions per tensor per tile
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

#define LDS __attribute__((address_space(3)))
typedef const LDS unsigned char* LdsBytes;  // operand reads address LDS directly

// Swizzle of the query-row tiles of the dk/dv backward kernel (Q' and dO,
// 64 rows), read two ways by 16x16x32 operands: as rows (the 16 lanes of a
// ds_read_b128 read one logical chunk of rows {8a + 4b + j : a, j in 0..3})
// and transposed (a ds_read_b64_tr_b16 per 16-lane group g reads rows
// 8g .. 8g+3 x 32 bytes). It depends on row bits 0, 1, 3 and 4 only: a lane's
// second transposing load is 4 rows down and the tile's two 32-row halves are
// addressed by a constant step. Picked among XOR swizzles of those bits by
// measuring SQ_LDS_BANK_CONFLICT for both patterns on gfx950: zero for both.
template <int HD>
__host__ __device__ constexpr int q_swz(int r) {
  return HD == 128 ? ((r & 1) | ((r & 1) << 1) | ((((r >> 1) ^ (r >> 4)) & 1) << 2) | (((r >> 3) & 1) << 3))
                   : ((r & 1) | (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2));
}
template <int HD>
__host__ __device__ constexpr int q_off(int r, int c) { return r * HD * 2 + ((c ^ q_swz<HD>(r)) << 4); }

// Swizzle of a K tile that the dq backward kernel reads both as 32x32x16
// A-operand rows (like K in the forward) and transposed (like V in the
// forward). Row bits 0 and 1 pick the 64-byte quarter (the transposing reads
// of rows r..r+3 land in different quarters), bits 2 and 3 the chunk inside
// it (16 rows of a row read spread over all 16 chunks). Measured with
// SQ_LDS_BANK_CONFLICT on gfx950: zero for both patterns. A lane's second
// transposing load (4 rows down) sees bit 0 of the swizzle flipped, i.e. its
// byte offset XOR kt_xor4. The 64-dim tile keeps the V swizzle.
template <int HD>
__host__ __device__ constexpr int kt_swz(int r) {
  return HD == 128 ? (((r >> 2) & 1) | (((r >> 3) & 1) << 1) | ((r & 1) << 2) | (((r >> 1) & 1) << 3)) : v_swz<HD>(r);
}
template <int HD>
__host__ __device__ constexpr int kt_off(int r, int c) { return r * HD * 2 + ((c ^ kt_swz<HD>(r)) << 4); }
template <int HD>
constexpr int kt_xor4() { return HD == 128 ? 16 : 0; }
template <int HD>
constexpr bool kt_rows_xor4() {
  for (int r = 0; r < 60; ++r)
    for (int c = 0; c < HD / 8; ++c)
      if ((r & 4) == 0 && kt_off<HD>(r + 4, c) != (kt_off<HD>(r, c) ^ kt_xor4<HD>()) + 4 * HD * 2) return false;
  return true;
}
static_assert(kt_rows_xor4<64>() && kt_rows_xor4<128>(), "K-tile swizzle: 4 rows down is XOR kt_xor4 plus 4 rows");

enum Swz { SWZ_K = 0, SWZ_V = 1, SWZ_Q = 2, SWZ_KT = 3 };
template <int HD, int KIND>
__host__ __device__ constexpr int swz(int r) {
  return KIND == SWZ_K ? k_swz<HD>(r) : (KIND == SWZ_V ? v_swz<HD>(r) : (KIND == SWZ_Q ? q_swz<HD>(r) : kt_swz<HD>(r)));
}

// Direct global -> LDS staging of one 64-row tile of two tensors (K/V, or Q'/dO
// in the backward), with no registers in between. Wave w of NWAVES issues wave
// instructions q = w*DMA/NWAVES .. of 1 KiB each per tensor; lane l of
// instruction q fills LDS bytes 1024q + 16l, i.e. row r = (1024q + 16l) / (2hd)
// at physical chunk pc, so it fetches the logical chunk pc ^ swz(r) of that row
// (SW0 / SW1 pick the swizzle of each tensor). The buffer descriptor starts at
// the tile and ends at the slab end: rows at or past T are written as zeros.
template <int HD, int NWAVES, int SW0 = SWZ_K, int SW1 = SWZ_V>
struct Dma {
  using C = Cfg<HD>;
  static constexpr int PER_WAVE = C::DMA / NWAVES;
  static_assert(C::DMA % NWAVES == 0, "every wave issues the same share of a tile");
  int koff[PER_WAVE];  // per-lane source byte offsets within the tile
  int voff[PER_WAVE];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int p = 1024 * (wave * PER_WAVE + i) + 16 * lane;
      const int r = p / (HD * 2), pc = (p % (HD * 2)) / 16;
      koff[i] = (r * HD + (pc ^ swz<HD, SW0>(r)) * 8) * 2;
      voff[i] = (r * HD + (pc ^ swz<HD, SW1>(r)) * 8) * 2;
    }
  }

  // Tile kt of both tensors, the first into kdst and the second into vdst.
  __device__ __forceinline__ void issue(const uint16_t* Kg, const uint16_t* Vg, int kt, int T, unsigned char* kdst,
                                        unsigned char* vdst, int wave) const {
    const int bytes = (T - kt * BN) * HD * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg + (long)kt * BN * HD, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg + (long)kt * BN * HD, bytes);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = wave * PER_WAVE + i;
#if defined(__HIP_DEVICE_COMPILE__)  // (the host pass drops the kernel stubs of later instantiations otherwise)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LDS void*)(kdst + 1024 * q), 16, koff[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LDS void*)(vdst + 1024 * q), 16, voff[i], 0, 0, 0);
#endif
    }
  }
  // Both tiles into one stage: the first tensor, then the second.
  __device__ __forceinline__ void issue(const uint16_t* Kg, const uint16_t* Vg, int kt, int T, unsigned char* stage,
                                        int wave) const {
    issue(Kg, Vg, kt, T, stage, stage + C::K_BYTES, wave);
  }
};

}  // namespace tile
}  // namespace attn
