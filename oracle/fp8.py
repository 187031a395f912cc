"""CPU oracle for a KV cache held in 8-bit floats (test infrastructure only).

TEST INFRASTRUCTURE ONLY, like oracle.attention: the plain fp64 definition,
imported only by the tests, the smoke check and the benchmark's CPU-baseline
leg; it shares nothing with the HIP path.

"Build a Transformer Self-Attention Block from Scratch in Pure Python" puts
int8 / fp8 representations on its roadmap as the next lever on the memory
bandwidth that grouped-query attention already cuts, and "Building a
Transformer from Scratch" tabulates the memory effect of 8-bit storage. The
pages fix no format; the reading taken here (and by the HIP path):

* the cache stores K and V as OCP FP8 E4M3 codes: 1 sign bit, 4 exponent bits
  with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
  m * 2^-9; there are no infinities and the two codes with all exponent and
  mantissa bits set are NaN, so the largest finite magnitude is 448;
* a cached value is code_value * scale, with one fp32 scale for all of K and
  one for all of V (per call);
* writing a value x stores the code nearest to x / scale after clamping to
  [-448, 448], ties to the code whose mantissa is even; the sign bit is the
  sign bit of x / scale (so -0.0 keeps it).

A decode step is then the decode of oracle.attention over the dequantized
cache, where the new token's rotated key and its value are first written
(quantized) to slot L and read back like every other slot.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import _attend, alibi_slopes, apply_rope

E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """The value of each of the 256 codes (NaN for the two NaN codes), from the
    bit layout: sign, 4-bit exponent field e (bias 7), 3-bit mantissa m."""
    vals = np.empty(256)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = math.nan
        elif e == 0:
            vals[code] = s * m * 2.0 ** -9
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def e4m3_decode(codes) -> np.ndarray:
    """Values of an array of uint8 codes (fp64)."""
    return e4m3_values()[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Codes of x: clamp |x| to 448, round to the nearest finite magnitude, ties
    to even mantissa, sign bit copied from x."""
    x = np.asarray(x, dtype=np.float64)
    mags = e4m3_values()[:0x7F]            # codes 0x00 .. 0x7e, increasing magnitudes
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(mags, a, side="left")          # first magnitude >= a
    hi = np.minimum(hi, len(mags) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - mags[lo]
    dhi = mags[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == mags[hi], hi, code).astype(np.uint8)   # exact hits
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def attention_decode_fp8(q, k_new, v_new, k_codes, v_codes, cache_lens, k_scale: float, v_scale: float, *,
                         rope_base: float = 10000.0, alibi: int = 0, batch=None):
    """One decode step over an fp8 cache.

    q [B,H,hd], k_new/v_new [B,KV,hd] (pre-rotation); k_codes/v_codes
    [B,KV,Lmax,hd] uint8 E4M3 codes of the already-rotated keys and the values
    (scaled by k_scale / v_scale). The new key is rotated at L = cache_lens[b],
    quantized with k_scale and stored at slot L, the value likewise with
    v_scale; the query (rotated at L) attends slots 0..L of the dequantized
    cache. Returns (out [B,H,hd], lse [B,H], k_slot_codes [B,KV,hd],
    v_slot_codes [B,KV,hd], k_slot_pre [B,KV,hd], v_slot_pre [B,KV,hd]) where
    *_pre are the values (divided by the scale) that were rounded to the slot
    codes."""
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    B, H, hd = q.shape
    KV = k_new.shape[1]
    group = H // KV
    scale = 1.0 / math.sqrt(hd)
    slopes = alibi_slopes(H, alibi)
    bs = list(range(B)) if batch is None else [int(b) for b in batch]
    lens = np.asarray(cache_lens)
    out = np.empty((len(bs), H, hd))
    lse = np.empty((len(bs), H))
    k_slot = np.empty((len(bs), KV, hd), dtype=np.uint8)
    v_slot = np.empty((len(bs), KV, hd), dtype=np.uint8)
    k_pre = np.empty((len(bs), KV, hd))
    v_pre = np.empty((len(bs), KV, hd))
    for n, b in enumerate(bs):
        L = int(lens[b])
        kidx = np.arange(L + 1)
        for g in range(KV):
            k_pre[n, g] = apply_rope(k_new[b, g][None], [L], rope_base)[0] / k_scale
            v_pre[n, g] = v_new[b, g] / v_scale
            k_slot[n, g] = e4m3_encode(k_pre[n, g])
            v_slot[n, g] = e4m3_encode(v_pre[n, g])
            # slots 0..L as stored, dequantized
            keys = e4m3_decode(np.concatenate([np.asarray(k_codes[b, g, :L]), k_slot[n, g][None]], axis=0)) * k_scale
            vals = e4m3_decode(np.concatenate([np.asarray(v_codes[b, g, :L]), v_slot[n, g][None]], axis=0)) * v_scale
            for h in range(g * group, (g + 1) * group):
                qr = apply_rope(q[b, h][None], [L], rope_base)
                o, l = _attend(qr, keys, vals, np.array([L]), kidx, True, slopes[h], scale)
                out[n, h] = o[0]
                lse[n, h] = l[0]
    return out, lse, k_slot, v_slot, k_pre, v_pre
