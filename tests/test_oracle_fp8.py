"""Pins for the fp8 (OCP E4M3) KV-cache oracle (CPU only).

The format and the rounding are pinned to torch's own float8_e4m3fn type (a
library routine implementing the OCP format), the decode step to the separately
pinned fp64 decode of oracle.attention on the dequantized cache.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention_decode, attention_decode_fp8, e4m3_decode, e4m3_encode, e4m3_values



def torch_decode(codes):
    return torch.tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def torch_encode(x):
    """torch rounds to nearest even but turns |x| > 464 into NaN: clamp first. Its
    conversion goes through fp32, so callers pass fp32-representable values."""
    x = np.clip(np.asarray(x, dtype=np.float64), -448.0, 448.0)
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)
    return torch.tensor(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_table_matches_torch():
    v = e4m3_values()
    t = torch_decode(np.arange(256))
    assert np.array_equal(np.isnan(v), np.isnan(t))
    assert np.array_equal(v[~np.isnan(v)], t[~np.isnan(t)])


def test_format_landmarks():
    v = e4m3_values()
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0           # largest finite
    assert v[0x01] == 2.0 ** -9                              # smallest subnormal
    assert v[0x08] == 2.0 ** -6 and v[0x07] == 7 * 2.0 ** -9  # smallest normal, largest subnormal
    assert v[0x38] == 1.0 and v[0xB8] == -1.0
    assert [c for c in range(256) if math.isnan(v[c])] == [0x7F, 0xFF]
    assert np.all(np.diff(v[:0x7F]) > 0)                    # magnitudes increase with the code


def test_encode_matches_torch_rounding():
    rng = np.random.default_rng(3)
    v = e4m3_values()
    mags = v[:0x7F]
    mids = (mags[1:] + mags[:-1]) / 2                       # every tie
    x = np.concatenate([rng.normal(size=20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 300.0)]
                       + [mags, -mags, mids, -mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20),
                          [0.0, -0.0, 448.0, 449.0, 464.0, 465.0, 1e6, -1e6, math.inf, -math.inf]])
    x = x.astype(np.float32).astype(np.float64)
    assert np.array_equal(e4m3_encode(x), torch_encode(x))


def test_encode_round_trip_and_ties_to_even():
    v = e4m3_values()
    finite = [c for c in range(256) if not math.isnan(v[c])]
    assert np.array_equal(e4m3_encode(v[finite]), np.array(finite, dtype=np.uint8))
    # 1 + 1/16 is halfway between 1 (code 0x38, even mantissa) and 1.125 (0x39)
    assert e4m3_encode(1.0 + 1 / 16) == 0x38
    assert e4m3_encode(1.125 + 1 / 16) == 0x3A
    assert e4m3_encode(2.0 ** -10) == 0x00 and e4m3_encode(3 * 2.0 ** -10) == 0x02   # subnormal ties


def _grid_case(seed, B=3, H=8, KV=2, hd=16, lens=(0, 5, 13), lmax=16, k_scale=0.125, v_scale=0.0625):
    rng = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    kc = rng.choice(finite, size=(B, KV, lmax, hd)).astype(np.uint8)
    vc = rng.choice(finite, size=(B, KV, lmax, hd)).astype(np.uint8)
    q = rng.normal(size=(B, H, hd))
    kn_codes = rng.choice(finite, size=(B, KV, hd)).astype(np.uint8)
    vn_codes = rng.choice(finite, size=(B, KV, hd)).astype(np.uint8)
    return q, kc, vc, kn_codes, vn_codes, np.array(lens, dtype=np.int32), k_scale, v_scale


@pytest.mark.parametrize("alibi", [0, 1])
def test_decode_equals_plain_decode_on_the_dequantized_cache(alibi):
    """Without RoPE and with new K/V already on the fp8 grid (times the scales),
    quantization is exact, so the fp8 step must equal the plain decode of the
    dequantized cache (a separately pinned routine)."""
    q, kc, vc, knc, vnc, lens, ks, vs = _grid_case(7)
    k_new = e4m3_decode(knc) * ks
    v_new = e4m3_decode(vnc) * vs
    out, lse, k_slot, v_slot, _, _ = attention_decode_fp8(q, k_new, v_new, kc, vc, lens, ks, vs, rope_base=0.0,
                                                          alibi=alibi)
    ref, ref_lse, _, _ = attention_decode(q, k_new, v_new, e4m3_decode(kc) * ks, e4m3_decode(vc) * vs, lens,
                                          rope_base=0.0, alibi=alibi)
    assert np.array_equal(k_slot, knc) and np.array_equal(v_slot, vnc)
    assert np.abs(out - ref).max() <= 1e-13 and np.abs(lse - ref_lse).max() <= 1e-13


def test_new_slot_is_the_rounded_rotated_key():
    """With RoPE the stored key is R(L) k_new / k_scale rounded by torch's float8 type."""
    q, kc, vc, _, _, lens, ks, vs = _grid_case(8)
    rng = np.random.default_rng(9)
    k_new = rng.normal(size=(3, 2, 16))
    v_new = rng.normal(size=(3, 2, 16))
    out, lse, k_slot, v_slot, k_pre, v_pre = attention_decode_fp8(q, k_new, v_new, kc, vc, lens, ks, vs,
                                                                  rope_base=10000.0)
    for b, L in enumerate(lens):
        # rotation by complex multiplication, written out independently of the oracle
        z = k_new[b, :, 0::2] + 1j * k_new[b, :, 1::2]
        theta = 10000.0 ** (-np.arange(8) * 2 / 16)
        zr = z * np.exp(1j * L * theta)
        kr = np.empty_like(k_new[b])
        kr[:, 0::2], kr[:, 1::2] = zr.real, zr.imag
        assert np.allclose(k_pre[b], kr / ks, rtol=0, atol=1e-12)
        # (torch's conversion rounds to fp32 first; these random values sit far from any tie)
        kf = (kr / ks).astype(np.float32).astype(np.float64)
        vf = (v_new[b] / vs).astype(np.float32).astype(np.float64)
        assert np.array_equal(k_slot[b], torch_encode(kf))
        assert np.array_equal(v_slot[b], torch_encode(vf))
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_quantization_error_is_bounded():
    """Caches quantized from exact values: the output moves by at most the
    values' rounding error (relative 2^-4 per E4M3 value, normal range)."""
    rng = np.random.default_rng(10)
    B, H, KV, hd, L = 2, 4, 1, 32, 50
    kx = rng.normal(size=(B, KV, L + 1, hd))
    vx = rng.normal(size=(B, KV, L + 1, hd))
    q = rng.normal(size=(B, H, hd)) * 0.3
    ks = vs = 1 / 64
    lens = np.array([L, L], dtype=np.int32)
    out, _, _, _, _, _ = attention_decode_fp8(q, kx[:, :, L], vx[:, :, L], e4m3_encode(kx / ks), e4m3_encode(vx / vs),
                                              lens, ks, vs, rope_base=0.0)
    ref, _, _, _ = attention_decode(q, kx[:, :, L], vx[:, :, L], kx, vx, lens, rope_base=0.0)
    assert 0 < np.abs(out - ref).max() <= 2.0 ** -4 * 4
