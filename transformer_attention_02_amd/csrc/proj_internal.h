// Arguments of the projection GEMMs either side of attention (the fused QKV
// projection with its rotary / head-split / cache-write epilogue, and the
// output projection with the head merge folded into its operand loads).
#pragma once

#include "attn_internal.h"

namespace attn {

enum ProjMode { PROJ_QKV = 0, PROJ_QKV_CACHE = 1, PROJ_OUT = 2 };

// C[M, N] = A[M, K] W[N, K]^T with rows m = b*T + t.
struct ProjArgs {
  const void* a;            // x [M, K] (QKV modes) or o [B, H, T, hd] (PROJ_OUT), bf16
  const void* w;            // [N, K] bf16, row-major (nn.Linear weight)
  int M, N, K;
  int T, H, KV, hd;
  unsigned a_bytes;         // bytes of a (< 2^31, the buffer-descriptor range)
  unsigned w_bytes;         // bytes of w (< 2^31)
  // QKV epilogue: column n < H*hd is query head n/hd, then KV key heads, then KV value heads
  void* q;                  // [B, H, T, hd]
  void* k;                  // [B, KV, T, hd] (PROJ_QKV)
  void* v;                  // [B, KV, T, hd] (PROJ_QKV)
  void* k_cache;            // [B, KV, Lmax, hd] (PROJ_QKV_CACHE)
  void* v_cache;
  const int32_t* lens;      // [B] (PROJ_QKV_CACHE): token t of sequence b at slot lens[b] + t
  int Lmax;
  int pos0;                 // PROJ_QKV: token t at position pos0 + t
  int rope;
  RopeFreqs freqs;
  // PROJ_OUT epilogue
  void* y;                  // [M, N]
  int out_bf16;
};

hipError_t launch_proj(const ProjArgs& a, int mode, hipStream_t s, const TimingHook& tm);

}  // namespace attn
