"""CPU oracle for the projections either side of attention (test infrastructure only).

TEST INFRASTRUCTURE ONLY, like oracle.attention: the plain fp64 definition,
imported only by the tests, the smoke check and the benchmark's CPU-baseline
leg; it shares nothing with the HIP path.

"Building Grouped-Query Attention with RoPE and Flash Attention from Scratch"
(Architecture Overview and Step 4) wraps the attention in a module with an
input projection that emits q, k and v (fewer K/V heads than query heads),
a rotary embedding of q and k, and an output projection that mixes the heads
back into the model dimension. Written out for x [B, T, D]:

    q = (x W_q^T).view(B, T, H,  hd).transpose(1, 2)      W_q [H hd,  D]
    k = (x W_k^T).view(B, T, KV, hd).transpose(1, 2)      W_k [KV hd, D]
    v = (x W_v^T).view(B, T, KV, hd).transpose(1, 2)      W_v [KV hd, D]
    q, k = RoPE(q), RoPE(k)
    y = out.transpose(1, 2).reshape(B, T, H hd) W_o^T     W_o [D, H hd]

The weights are nn.Linear weights ([out_features, in_features], y = x W^T,
no bias, as on the page). The fused weight w_qkv stacks the rows of W_q, W_k
and W_v in that order (the page's comment on one fused QKV projection); so
column n of x w_qkv^T is query head n // hd when n < H hd, then key head, then
value head, dim n % hd.

Readings taken here:
* The rotation is the interleaved-pair RoPE of oracle.attention.apply_rope
  (the same convention every other path of this library uses); token t sits
  at position pos0 + t. rope_base 0 means no rotation.
* KV-cache write (lab Exercise 2 of "Write attention from scratch"; the
  roadmap's pre-allocated cache written by position on the GQA page): for
  tokens appended to a cache, token t of sequence b sits at position
  cache_lens[b] + t; its rotated key and its value go to that slot of the
  cache. A sequence whose slots would fall outside [0, Lmax) gets NaN queries
  and its cache is left as it was.
"""
from __future__ import annotations

import numpy as np

from .attention import apply_rope


def _split_heads(y, heads: int, hd: int):
    """[B, T, heads*hd] -> [B, heads, T, hd] (the view + transpose of the page)."""
    B, T, _ = y.shape
    return y.reshape(B, T, heads, hd).transpose(0, 2, 1, 3).copy()


def qkv_projection(x, w_qkv, *, H: int, KV: int, hd: int, pos0: int = 0, rope_base: float = 10000.0,
                   positions=None):
    """Input projection and rotary embedding.

    x [B,T,D], w_qkv [(H+2KV)*hd, D]. Returns (q [B,H,T,hd], k [B,KV,T,hd],
    v [B,KV,T,hd]) in fp64, q and k rotated at position pos0 + t, or at
    positions[b] + t when ``positions`` (one start per sequence) is given.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_qkv, dtype=np.float64)
    B, T, D = x.shape
    if w.shape != ((H + 2 * KV) * hd, D):
        raise ValueError("w_qkv must be [(H + 2 KV) hd, D]")
    y = x @ w.T                                            # [B, T, (H+2KV) hd]
    q = _split_heads(y[..., :H * hd], H, hd)
    k = _split_heads(y[..., H * hd:(H + KV) * hd], KV, hd)
    v = _split_heads(y[..., (H + KV) * hd:], KV, hd)
    if rope_base:
        for b in range(B):
            start = pos0 if positions is None else int(positions[b])
            pos = np.arange(T) + start
            q[b] = apply_rope(q[b], pos, rope_base)
            k[b] = apply_rope(k[b], pos, rope_base)
    return q, k, v


def qkv_projection_to_cache(x, w_qkv, k_cache, v_cache, cache_lens, *, H: int, KV: int, hd: int,
                            rope_base: float = 10000.0):
    """The projection for T tokens appended to a KV cache.

    k_cache / v_cache [B,KV,Lmax,hd]; token t of sequence b sits at position
    cache_lens[b] + t and its key (rotated) and value are written to that slot.
    Returns (q [B,H,T,hd], k_cache', v_cache') with the updated caches (fp64
    copies); sequences whose slots leave [0, Lmax) get NaN queries and keep
    their cache.
    """
    x = np.asarray(x, dtype=np.float64)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    lens = np.asarray(cache_lens, dtype=np.int64)
    B, T, _ = x.shape
    Lmax = kc.shape[2]
    q, k, v = qkv_projection(x, w_qkv, H=H, KV=KV, hd=hd, rope_base=rope_base, positions=lens)
    for b in range(B):
        L = int(lens[b])
        if L < 0 or L + T > Lmax:
            q[b] = np.nan
            continue
        kc[b, :, L:L + T] = k[b]
        vc[b, :, L:L + T] = v[b]
    return q, kc, vc


def out_projection(o, w_o):
    """y [B,T,D] = o.transpose(1, 2).reshape(B, T, H*hd) W_o^T; o [B,H,T,hd], w_o [D, H*hd]."""
    o = np.asarray(o, dtype=np.float64)
    w = np.asarray(w_o, dtype=np.float64)
    B, H, T, hd = o.shape
    if w.shape[1] != H * hd:
        raise ValueError("w_o must be [D, H hd]")
    return o.transpose(0, 2, 1, 3).reshape(B, T, H * hd) @ w.T


def proj_flops(M: int, N: int, K: int) -> float:
    """Algorithmic flops of one projection: M x N outputs, K multiply-adds each."""
    return 2.0 * M * N * K
