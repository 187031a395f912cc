"""CPU oracle for causal grouped-query attention with rotary embeddings and ALiBi.

TEST INFRASTRUCTURE ONLY. This is the plain, slow, obviously correct fp64
definition of what the attention path computes. It exists to check the HIP
library; only the tests, the smoke check and the benchmark's CPU-baseline leg
may import it. It shares no code, tables or helpers with the HIP path and it
never imports the package that holds it.

What is computed (all in fp64 from the exact values the GPU receives):

* Rotary embedding, interleaved pairs ("Write attention from scratch", the lab
  listing's rope function; frequency schedule theta_i = base^(-2i/hd) as on
  every page): pair (2i, 2i+1) of a vector at position p is rotated by the
  angle p * theta_i. Q and K are rotated, V is not (lab Exercise 1 explains why
  rotating V breaks the relative-position property).
* Scores s_ij = <q'_i, k'_j> / sqrt(hd) ("Building a Transformer from Scratch",
  Part 1, the scaled dot-product equation), plus an ALiBi bias
  -slope_h * |i - j| added after the scaling ("Building a Multi-Head
  Self-Attention Block with RoPE and ALiBi", Architecture Overview formula
  softmax(QK^T/sqrt(d_k) + M) and Step 3's distance-times-slope bias).
* Causal visibility j <= i (the lab listing's lower-triangular mask; "Build a
  Transformer Self-Attention Block ... in Pure Python", Step 4). Masked keys
  get exactly zero weight: they are simply left out of the softmax.
* Stable softmax (subtract the row max, exponentiate, normalise; "Pure Python"
  page Step 1) and the weighted sum of V rows.
* Grouped-query sharing: query head h reads key/value head h // (H / KV), the
  consecutive grouping that np.repeat / repeat_interleave produce (lab listing;
  "Building Grouped-Query Attention with RoPE and Flash Attention", Step 3).
* KV-cache decode: a new token at position L = cache length attends cached keys
  0..L-1 (already rotated) plus its own key rotated at L (lab Exercise 2: the
  incremental result must equal the full computation; "Building Grouped-Query
  Attention ...", roadmap item on a pre-allocated cache written by position).
* Chunked prefill: a chunk of Tq queries that are tokens q_offset ..
  q_offset+Tq-1 of a key sequence of Tk tokens (the chunk's own keys included)
  attends with the same causal test on token indices. Processing a prompt
  chunk by chunk must reproduce the full computation (lab Exercise 2 with
  chunks instead of single tokens).
* Sliding window (the lab's Exercise 3, and the sliding-window mode on the
  roadmap of "Building Grouped-Query Attention ..."): with a window of W tokens
  the query at token i sees keys j with i - W < j <= i, i.e. itself and the
  W - 1 tokens before it.

The tiled online softmax that the GPU runs is an exact rearrangement of this
definition (the recurrences of "Building a Transformer from Scratch", Part 3,
and Step 3 of the Flash-Attention page), so the oracle is the definition, not
the tiling.

Every function here is pinned by the CPU tests (brute force with complex
rotations, a library softmax-attention routine, the lab's two printed
properties, closed forms and invariants).
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)

ALIBI_NONE = 0
ALIBI_GEOMETRIC = 1   # slope_h = 2^(-8(h+1)/H)
ALIBI_PAGE1 = 2       # slope_h = 2^(-2(h+1)/H), the heuristic printed in Step 1 of the multi-head page


def rope_inv_freq(hd: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/hd), i = 0 .. hd/2-1, in fp64."""
    i = np.arange(hd // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / hd)


def apply_rope(x: np.ndarray, positions, base: float) -> np.ndarray:
    """Rotate interleaved pairs of the last axis of ``x`` ([..., T, hd]).

    ``positions`` has length T (one position per row). Pair (2i, 2i+1) at
    position p becomes (x0 cos a - x1 sin a, x0 sin a + x1 cos a), a = p*theta_i.
    ``base == 0`` means no rotation.
    """
    x = np.asarray(x, dtype=np.float64)
    if base == 0:
        return x.copy()
    hd = x.shape[-1]
    if hd % 2:
        raise ValueError("rotary embedding needs an even head dimension")
    pos = np.asarray(positions, dtype=np.float64).reshape(-1, 1)
    ang = pos * rope_inv_freq(hd, base)[None, :]          # [T, hd/2]
    c, s = np.cos(ang), np.sin(ang)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def alibi_slopes(H: int, kind: int) -> np.ndarray:
    """Per-head ALiBi slopes (fp64). kind 0 -> zeros."""
    h = np.arange(H, dtype=np.float64)
    if kind == ALIBI_NONE:
        return np.zeros(H)
    if kind == ALIBI_GEOMETRIC:
        return np.power(2.0, -8.0 * (h + 1.0) / H)
    if kind == ALIBI_PAGE1:
        return np.power(2.0, -2.0 * (h + 1.0) / H)
    raise ValueError(f"unknown ALiBi kind {kind}")


def _attend(qr, kr, v, q_idx, k_idx, causal, slope, scale, window=0):
    """Softmax attention of rotated query rows ``qr`` [n, hd] over keys ``kr`` [m, hd].

    ``q_idx``/``k_idx`` are the token indices used for the causal test, the
    sliding window (``window`` > 0: keys within the last ``window`` tokens up to
    and including the query's) and the ALiBi distance. Returns (out [n, hd],
    lse [n]) with lse = log sum_j exp(s_ij) over the visible keys.
    """
    s = (qr @ kr.T) * scale                                   # [n, m]
    dist = q_idx[:, None].astype(np.float64) - k_idx[None, :].astype(np.float64)
    if slope != 0.0:
        s = s - slope * np.abs(dist)
    out = np.empty((qr.shape[0], v.shape[1]))
    lse = np.empty(qr.shape[0])
    for r in range(qr.shape[0]):
        row = s[r]
        vis = (k_idx <= q_idx[r]) if causal else np.ones(len(k_idx), dtype=bool)
        if window:
            vis &= k_idx > q_idx[r] - window
        sv = row[vis]
        m = sv.max()
        e = np.exp(sv - m)
        z = e.sum()
        out[r] = (e / z) @ v[vis]
        lse[r] = m + math.log(z)
    return out, lse


def attention_prefill(q, k, v, *, pos0: int = 0, rope_base: float = 10000.0, causal: bool = True,
                      alibi: int = ALIBI_NONE, rows=None, q_offset: int = 0, window: int = 0):
    """Attention forward over a sequence, or over a chunk of its queries.

    q [B,H,Tq,hd]; k, v [B,KV,Tk,hd] (pre-rotation). Key token j sits at
    position pos0 + j; query row i is token q_offset + i (position
    pos0 + q_offset + i), and q_offset + Tq <= Tk (the chunk's own keys are part
    of k). ``window`` > 0 (causal only) limits each query to its last
    ``window`` tokens. Returns (out [B,H,Tq,hd], lse [B,H,Tq]) in fp64.

    ``rows`` optionally restricts the computation to a list of (b, h, i)
    triples; the result is then (out [n, hd], lse [n]) in that order.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Tq, hd = q.shape
    KV, Tk = k.shape[1], k.shape[2]
    if H % KV:
        raise ValueError("query heads must be a multiple of key/value heads")
    if q_offset < 0 or q_offset + Tq > Tk:
        raise ValueError("the query chunk must lie inside the key sequence")
    if window < 0 or (window and not causal):
        raise ValueError("a sliding window needs causal attention and a positive width")
    group = H // KV
    scale = 1.0 / math.sqrt(hd)
    slopes = alibi_slopes(H, alibi)
    positions = pos0 + np.arange(Tk)
    idx = np.arange(Tk)
    q_tok = q_offset + np.arange(Tq)

    if rows is not None:
        rows = [tuple(int(t) for t in r) for r in rows]
        out = np.empty((len(rows), hd))
        lse = np.empty(len(rows))
        by_head = {}
        for n, (b, h, i) in enumerate(rows):
            by_head.setdefault((b, h), []).append((n, i))
        for (b, h), lst in by_head.items():
            g = h // group
            qi = np.array([i for _, i in lst])
            qr = apply_rope(q[b, h, qi], positions[q_tok[qi]], rope_base)
            kr = apply_rope(k[b, g], positions, rope_base)
            o, l = _attend(qr, kr, v[b, g], q_tok[qi], idx, causal, slopes[h], scale, window)
            for j, (n, _) in enumerate(lst):
                out[n] = o[j]
                lse[n] = l[j]
        return out, lse

    out = np.empty((B, H, Tq, hd))
    lse = np.empty((B, H, Tq))
    for b in range(B):
        for g in range(KV):
            kr = apply_rope(k[b, g], positions, rope_base)
            for h in range(g * group, (g + 1) * group):
                qr = apply_rope(q[b, h], positions[q_tok], rope_base)
                out[b, h], lse[b, h] = _attend(qr, kr, v[b, g], q_tok, idx, causal, slopes[h], scale, window)
    return out, lse


def attention_decode(q, k_new, v_new, k_cache, v_cache, cache_lens, *, rope_base: float = 10000.0,
                     alibi: int = ALIBI_NONE, batch=None):
    """One decode step per sequence with a pre-allocated cache.

    q [B,H,hd], k_new/v_new [B,KV,hd] are the new token's pre-rotation vectors;
    k_cache/v_cache [B,KV,Lmax,hd] hold already-rotated keys and values at slots
    0..L-1, L = cache_lens[b]. The new token sits at position L: its key is
    rotated at L and appended at slot L, and the query (rotated at L) attends
    slots 0..L. Returns (out [B,H,hd], lse [B,H], k_slot [B,KV,hd], v_slot)
    where k_slot/v_slot are the values written at slot L.

    ``batch`` optionally restricts the computation to some sequence indices;
    the outputs then follow that order.
    """
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    B, H, hd = q.shape
    KV = k_new.shape[1]
    group = H // KV
    scale = 1.0 / math.sqrt(hd)
    slopes = alibi_slopes(H, alibi)
    bs = list(range(B)) if batch is None else [int(b) for b in batch]
    out = np.empty((len(bs), H, hd))
    lse = np.empty((len(bs), H))
    k_slot = np.empty((len(bs), KV, hd))
    v_slot = np.empty((len(bs), KV, hd))
    for n, b in enumerate(bs):
        L = int(cache_lens[b])
        kidx = np.arange(L + 1)
        for g in range(KV):
            kn = apply_rope(k_new[b, g][None], [L], rope_base)[0]
            keys = np.concatenate([np.asarray(k_cache[b, g, :L], dtype=np.float64), kn[None]], axis=0)
            vals = np.concatenate([np.asarray(v_cache[b, g, :L], dtype=np.float64), v_new[b, g][None]], axis=0)
            k_slot[n, g] = kn
            v_slot[n, g] = v_new[b, g]
            for h in range(g * group, (g + 1) * group):
                qr = apply_rope(q[b, h][None], [L], rope_base)
                o, l = _attend(qr, keys, vals, np.array([L]), kidx, True, slopes[h], scale)
                out[n, h] = o[0]
                lse[n, h] = l[0]
    return out, lse, k_slot, v_slot


def attention_prefill_bwd(q, k, v, dout, *, pos0: int = 0, rope_base: float = 10000.0, causal: bool = True,
                          alibi: int = ALIBI_NONE):
    """Gradients of sum(out * dout) with respect to the pre-rotation q, k and v.

    The backward of the same definition (the gradient-flow checks of the
    multi-head and pure-Python pages, and the pure-Python page's finite-difference
    test, exercise exactly these derivatives). With the rotated q', k' and the
    softmax weights p_ij of each visible pair:
      dv_j  = sum_i p_ij dout_i                       (summed over the group's heads)
      dp_ij = <dout_i, v_j>
      ds_ij = p_ij (dp_ij - sum_l p_il dp_il)         (softmax derivative)
      dq'_i = scale sum_j ds_ij k'_j,   dk'_j = scale sum_i ds_ij q'_i
    and the rotation is orthogonal, so dq = R(p_i)^T dq' = R(-p_i) dq' (same for
    k). The ALiBi bias does not depend on q, k or v. q, k, v, dout as for
    attention_prefill (Tq = Tk = T); returns (dq [B,H,T,hd], dk [B,KV,T,hd],
    dv [B,KV,T,hd]) in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, H, T, hd = q.shape
    KV = k.shape[1]
    if H % KV:
        raise ValueError("query heads must be a multiple of key/value heads")
    group = H // KV
    scale = 1.0 / math.sqrt(hd)
    slopes = alibi_slopes(H, alibi)
    positions = pos0 + np.arange(T)
    idx = np.arange(T)
    vis = (idx[None, :] <= idx[:, None]) if causal else np.ones((T, T), dtype=bool)
    dist = np.abs(idx[:, None] - idx[None, :]).astype(np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for g in range(KV):
            kr = apply_rope(k[b, g], positions, rope_base)
            dkr = np.zeros((T, hd))
            for h in range(g * group, (g + 1) * group):
                qr = apply_rope(q[b, h], positions, rope_base)
                s = (qr @ kr.T) * scale - slopes[h] * dist
                s = np.where(vis, s, -np.inf)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                do = dout[b, h]
                dv[b, g] += p.T @ do
                dp = do @ v[b, g].T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, h] = apply_rope(ds @ kr * scale, -positions, rope_base)
                dkr += ds.T @ qr * scale
            dk[b, g] = apply_rope(dkr, -positions, rope_base)
    return dq, dk, dv


def prefill_flops(B: int, H: int, T: int, hd: int, causal: bool = True) -> float:
    """Algorithmic flops of the forward: 2 contractions x 2 flops per visible (i, j) pair per dim."""
    pairs = T * (T + 1) / 2 if causal else T * T
    return 4.0 * B * H * hd * pairs


def kv_bytes_per_token(KV: int, hd: int, elem_bytes: int) -> int:
    """Cache bytes one token adds per layer: K and V, KV heads of hd elements."""
    return 2 * KV * hd * elem_bytes
