"""CPU oracle for latent-attention decode (test infrastructure only).

TEST INFRASTRUCTURE ONLY, like oracle.attention: the plain fp64 definition,
imported only by the tests, the smoke check and the benchmark's CPU-baseline
leg; it shares nothing with the HIP path.

Exercise 5 of "Write attention from scratch" replaces the key and value
projections with a down-projection of each token to a short latent vector and
per-head up-projections, and asks to fold the key up-projection into the
query and check that the scores do not change. Written out, for a token j
with latent c_j (d_c numbers, shared by every head) and query head h:

    k_hj = c_j W_uk[h],   v_hj = c_j W_uv[h]        (W_uk[h], W_uv[h]: d_c x hd)
    s_hj = <q_h, k_hj> / sqrt(hd) = <W_uk[h] q_h, c_j> / sqrt(hd)
    out_h = sum_j p_hj v_hj = (sum_j p_hj c_j) W_uv[h]

so a decode step needs only the latent cache: the folded query
q~_h = W_uk[h] q_h attends the latents directly and the weighted latent sum is
up-projected once per head. The reading taken here: the latent path carries
no rotary embedding (a position-dependent rotation of k_hj does not commute
with the fold, so the exercise's check holds only without it); ALiBi, being a
bias on the scores, is allowed. Decode is as in oracle.attention: the new
token at position L = cache length appends its latent at slot L and attends
slots 0..L.

attention_decode_latent is the definition above with explicit per-head keys
and values (no fold); fold_query is the fold on its own.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import _attend, alibi_slopes


def fold_query(q, w_uk) -> np.ndarray:
    """q~[b, h] = W_uk[h] q[b, h]: q [B,H,hd], w_uk [H,d_c,hd] -> [B,H,d_c]."""
    q = np.asarray(q, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    return np.einsum("hcd,bhd->bhc", w_uk, q)


def attention_decode_latent(q, c_new, c_cache, cache_lens, w_uk, w_uv, *, alibi: int = 0, batch=None):
    """One decode step over a latent cache.

    q [B,H,hd] (the new token's queries), c_new [B,d_c] (its latent),
    c_cache [B,Lmax,d_c] (latents at slots 0..L-1, L = cache_lens[b]),
    w_uk / w_uv [H,d_c,hd]. Keys and values of every head are formed
    explicitly from the latents (slot L holding c_new); scores are scaled by
    1/sqrt(hd). Returns (out [B,H,hd], lse [B,H], c_slot [B,d_c]) with c_slot
    the latent written at slot L.
    """
    q = np.asarray(q, dtype=np.float64)
    c_new = np.asarray(c_new, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    B, H, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    slopes = alibi_slopes(H, alibi)
    bs = list(range(B)) if batch is None else [int(b) for b in batch]
    lens = np.asarray(cache_lens)
    out = np.empty((len(bs), H, hd))
    lse = np.empty((len(bs), H))
    c_slot = np.empty((len(bs), c_new.shape[-1]))
    for n, b in enumerate(bs):
        L = int(lens[b])
        lat = np.concatenate([np.asarray(c_cache[b, :L], dtype=np.float64), c_new[b][None]], axis=0)  # [L+1, d_c]
        c_slot[n] = c_new[b]
        kidx = np.arange(L + 1)
        for h in range(H):
            keys = lat @ w_uk[h]        # [L+1, hd]
            vals = lat @ w_uv[h]
            o, l = _attend(q[b, h][None], keys, vals, np.array([L]), kidx, True, slopes[h], scale)
            out[n, h] = o[0]
            lse[n, h] = l[0]
    return out, lse, c_slot
