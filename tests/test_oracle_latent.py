"""Pins for the latent-attention decode oracle (CPU only)."""
import numpy as np
import pytest
import torch

from brute import brute_attention
from oracle import attention_decode, attention_decode_latent, fold_query


def _case(seed, B=3, H=4, hd=8, dc=8, lens=(0, 4, 9), lmax=10):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(B, H, hd))
    c_cache = rng.normal(size=(B, lmax, dc))
    c_new = rng.normal(size=(B, dc))
    w_uk = rng.normal(size=(H, dc, hd)) / np.sqrt(dc)
    w_uv = rng.normal(size=(H, dc, hd)) / np.sqrt(dc)
    return q, c_new, c_cache, np.array(lens, dtype=np.int32), w_uk, w_uv


def test_folded_scores_are_unchanged():
    """The lab's Exercise 5 check: <q, c W_uk> equals <W_uk q, c> for every head and token
    (here through torch's own matmul, in fp64)."""
    q, c_new, c_cache, lens, w_uk, w_uv = _case(1)
    qf = fold_query(q, w_uk)
    for b in range(q.shape[0]):
        lat = torch.tensor(c_cache[b])
        for h in range(q.shape[1]):
            s_explicit = (lat @ torch.tensor(w_uk[h])) @ torch.tensor(q[b, h])
            s_folded = lat @ torch.tensor(qf[b, h])
            assert torch.allclose(s_explicit, s_folded, rtol=0, atol=1e-13)


@pytest.mark.parametrize("alibi", [0, 1])
def test_latent_decode_reduces_to_gqa_decode(alibi):
    """With d_c = KV*hd and up-projections that select head h's KV block (and copy it), the
    latent cache is a plain K/V cache: the step must equal the pinned GQA decode without RoPE."""
    rng = np.random.default_rng(2)
    B, H, KV, hd, lmax = 2, 6, 2, 8, 12
    lens = np.array([5, 11], dtype=np.int32)
    dc = 2 * KV * hd                      # latent = [k of every KV head | v of every KV head]
    c_cache = rng.normal(size=(B, lmax, dc))
    c_new = rng.normal(size=(B, dc))
    q = rng.normal(size=(B, H, hd))
    w_uk = np.zeros((H, dc, hd))
    w_uv = np.zeros((H, dc, hd))
    g = H // KV
    for h in range(H):
        kv = h // g
        w_uk[h, kv * hd:(kv + 1) * hd] = np.eye(hd)
        w_uv[h, KV * hd + kv * hd:KV * hd + (kv + 1) * hd] = np.eye(hd)
    out, lse, c_slot = attention_decode_latent(q, c_new, c_cache, lens, w_uk, w_uv, alibi=alibi)
    k_cache = c_cache[:, :, :KV * hd].reshape(B, lmax, KV, hd).transpose(0, 2, 1, 3)
    v_cache = c_cache[:, :, KV * hd:].reshape(B, lmax, KV, hd).transpose(0, 2, 1, 3)
    k_new = c_new[:, :KV * hd].reshape(B, KV, hd)
    v_new = c_new[:, KV * hd:].reshape(B, KV, hd)
    ref, ref_lse, _, _ = attention_decode(q, k_new, v_new, k_cache, v_cache, lens, rope_base=0.0, alibi=alibi)
    assert np.abs(out - ref).max() <= 1e-13 and np.abs(lse - ref_lse).max() <= 1e-13
    assert np.array_equal(c_slot, c_new)


def test_zero_query_averages_the_latents():
    """q = 0: every visible slot weighs 1/(L+1), so out_h = mean_j(c_j) W_uv[h], lse = log(L+1)."""
    q, c_new, c_cache, lens, w_uk, w_uv = _case(3)
    q[:] = 0.0
    out, lse, _ = attention_decode_latent(q, c_new, c_cache, lens, w_uk, w_uv)
    for b, L in enumerate(lens):
        lat = np.concatenate([c_cache[b, :L], c_new[b][None]])
        for h in range(q.shape[1]):
            assert np.allclose(out[b, h], lat.mean(0) @ w_uv[h], rtol=0, atol=1e-13)
            assert abs(lse[b, h] - np.log(L + 1)) <= 1e-13


def test_latent_decode_is_the_lab_block_with_latent_projections():
    """The lab's attention written with the latent projections (no RoPE, as the fold needs):
    the last token's row of a causal block over all tokens, computed by the scalar brute force
    on the explicit per-head keys and values, equals a decode step whose cache holds the
    earlier tokens' latents."""
    rng = np.random.default_rng(0)
    T, d, H, dc = 6, 32, 4, 8
    hd = d // H
    x, wq, w_dkv, w_uk, w_uv = (rng.normal(size=shape) / np.sqrt(fan_in) for shape, fan_in in (
        ((T, d), 1.0), ((d, H * hd), d), ((d, dc), d), ((H, dc, hd), dc), ((H, dc, hd), dc)))
    c = x @ w_dkv                                                 # latents [T, dc]
    q = (x @ wq).reshape(T, H, hd).transpose(1, 0, 2)              # [H, T, hd]
    k = np.stack([c @ w_uk[h] for h in range(H)])                  # each head's keys and values
    v = np.stack([c @ w_uv[h] for h in range(H)])
    full, _ = brute_attention(q[None], k[None], v[None], 0, 0.0, True, 0)
    out, _, _ = attention_decode_latent(q[:, -1][None], c[-1][None], c[None, :-1], np.array([T - 1]), w_uk, w_uv)
    assert np.abs(out[0] - full[0, :, -1]).max() <= 1e-13
