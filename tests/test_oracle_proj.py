"""Pins for the projection oracle (CPU only).

Each test checks oracle.proj against something other than itself: torch's own
nn.Linear semantics and the page's view/transpose (in fp64), the rotary
embedding written as a complex multiplication, explicit index loops, the lab's
token-by-token KV-cache equivalence, the relative-position property of RoPE,
and the whole block against torch's scaled_dot_product_attention.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention_prefill, out_projection, qkv_projection, qkv_projection_to_cache


def _case(seed, B=2, T=5, H=4, KV=2, hd=8, D=None):
    rng = np.random.default_rng(seed)
    D = D or H * hd
    x = rng.normal(size=(B, T, D))
    w = rng.normal(size=((H + 2 * KV) * hd, D)) / math.sqrt(D)
    return x, w


def _torch_rope_complex(t, positions, base):
    """Interleaved pairs as complex numbers x0 + i x1, multiplied by e^{i p theta_i}."""
    hd = t.shape[-1]
    theta = base ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    ang = torch.as_tensor(positions, dtype=torch.float64)[:, None] * theta[None, :]
    z = torch.view_as_complex(t.reshape(*t.shape[:-1], hd // 2, 2).contiguous())
    return torch.view_as_real(z * torch.polar(torch.ones_like(ang), ang)).reshape(t.shape)


@pytest.mark.parametrize("rope_base,pos0", [(0.0, 0), (10000.0, 0), (500000.0, 37)])
def test_projection_matches_torch_linear_module(rope_base, pos0):
    """The page's forward: q_proj/k_proj/v_proj as nn.Linear (y = x W^T), view(B,T,heads,hd),
    transpose(1, 2), then RoPE of q and k (here the complex-number form)."""
    B, T, H, KV, hd = 2, 5, 4, 2, 8
    x, w = _case(1, B, T, H, KV, hd)
    q, k, v = qkv_projection(x, w, H=H, KV=KV, hd=hd, pos0=pos0, rope_base=rope_base)
    xt, wt = torch.tensor(x), torch.tensor(w)
    wq, wk, wv = wt[:H * hd], wt[H * hd:(H + KV) * hd], wt[(H + KV) * hd:]
    tq = F.linear(xt, wq).view(B, T, H, hd).transpose(1, 2)
    tk = F.linear(xt, wk).view(B, T, KV, hd).transpose(1, 2)
    tv = F.linear(xt, wv).view(B, T, KV, hd).transpose(1, 2)
    if rope_base:
        pos = np.arange(T) + pos0
        tq, tk = _torch_rope_complex(tq, pos, rope_base), _torch_rope_complex(tk, pos, rope_base)
    for mine, ref in ((q, tq), (k, tk), (v, tv)):
        assert np.abs(mine - ref.numpy()).max() <= 1e-12


def test_identity_weights_split_heads():
    """W_q = I, W_k = 2I (first KV*hd dims), W_v = 3I (next KV*hd dims), no rotation: every output
    element is the input element at [b, t, head*hd + d], read with explicit indices."""
    B, T, H, KV, hd = 2, 3, 4, 2, 4
    D = H * hd
    x = np.random.default_rng(2).normal(size=(B, T, D))
    w = np.zeros(((H + 2 * KV) * hd, D))
    w[:H * hd] = np.eye(D)
    for r in range(KV * hd):
        w[H * hd + r, r] = 2.0
        w[(H + KV) * hd + r, KV * hd + r] = 3.0
    q, k, v = qkv_projection(x, w, H=H, KV=KV, hd=hd, rope_base=0.0)
    for b in range(B):
        for t in range(T):
            for d in range(hd):
                for h in range(H):
                    assert q[b, h, t, d] == x[b, t, h * hd + d]
                for j in range(KV):
                    assert k[b, j, t, d] == 2.0 * x[b, t, j * hd + d]
                    assert v[b, j, t, d] == 3.0 * x[b, t, KV * hd + j * hd + d]


def test_cache_write_token_by_token_equals_full():
    """The lab's Exercise 2 for the projection: appending the tokens one at a time (T = 1, the
    position taken from the cache length) fills the cache with the full projection's k and v and
    yields its q rows."""
    B, T, H, KV, hd, Lmax = 2, 6, 4, 2, 8, 9
    x, w = _case(3, B, T, H, KV, hd)
    q, k, v = qkv_projection(x, w, H=H, KV=KV, hd=hd, rope_base=10000.0)
    kc = np.zeros((B, KV, Lmax, hd))
    vc = np.zeros((B, KV, Lmax, hd))
    for t in range(T):
        lens = np.full(B, t, dtype=np.int32)
        qt, kc, vc = qkv_projection_to_cache(x[:, t:t + 1], w, kc, vc, lens, H=H, KV=KV, hd=hd, rope_base=10000.0)
        assert np.abs(qt[:, :, 0] - q[:, :, t]).max() <= 1e-12
    assert np.abs(kc[:, :, :T] - k).max() <= 1e-12 and np.abs(vc[:, :, :T] - v).max() <= 1e-12
    assert not kc[:, :, T:].any() and not vc[:, :, T:].any()


def test_cache_write_chunk_at_offsets_and_bad_lengths():
    """A chunk of T tokens lands at slots L .. L+T-1 of each sequence (positions L + t); a sequence
    whose chunk would leave [0, Lmax) gets NaN queries and an untouched cache."""
    B, T, H, KV, hd, Lmax = 3, 3, 2, 1, 4, 8
    x, w = _case(4, B, T, H, KV, hd)
    lens = np.array([2, 6, -1], dtype=np.int32)          # 6 + 3 > 8 and -1 are out of range
    rng = np.random.default_rng(5)
    kc0, vc0 = rng.normal(size=(B, KV, Lmax, hd)), rng.normal(size=(B, KV, Lmax, hd))
    q, kc, vc = qkv_projection_to_cache(x, w, kc0, vc0, lens, H=H, KV=KV, hd=hd, rope_base=10000.0)
    q0, k0, v0 = qkv_projection(x[:1], w, H=H, KV=KV, hd=hd, pos0=2, rope_base=10000.0)
    assert np.abs(q[0] - q0[0]).max() <= 1e-12
    assert np.abs(kc[0, :, 2:5] - k0[0]).max() <= 1e-12 and np.abs(vc[0, :, 2:5] - v0[0]).max() <= 1e-12
    assert np.array_equal(kc[0, :, :2], kc0[0, :, :2]) and np.array_equal(kc[0, :, 5:], kc0[0, :, 5:])
    for b in (1, 2):
        assert np.isnan(q[b]).all()
        assert np.array_equal(kc[b], kc0[b]) and np.array_equal(vc[b], vc0[b])


def test_rope_scores_depend_on_relative_position_only():
    """Shifting every position by the same offset leaves every q.k score unchanged."""
    B, T, H, KV, hd = 1, 7, 2, 1, 8
    x, w = _case(6, B, T, H, KV, hd)
    q0, k0, _ = qkv_projection(x, w, H=H, KV=KV, hd=hd, pos0=0, rope_base=10000.0)
    q1, k1, _ = qkv_projection(x, w, H=H, KV=KV, hd=hd, pos0=1234, rope_base=10000.0)
    s0 = q0[0, 0] @ k0[0, 0].T
    s1 = q1[0, 0] @ k1[0, 0].T
    assert np.abs(s0 - s1).max() <= 1e-9
    assert np.abs(q0 - q1).max() > 1e-3                    # the rows themselves do move


def test_out_projection_matches_torch_linear_module():
    """out.transpose(1, 2).contiguous().view(B, T, H*hd), then o_proj as nn.Linear."""
    B, H, T, hd, D = 2, 4, 5, 8, 24
    rng = np.random.default_rng(7)
    o = rng.normal(size=(B, H, T, hd))
    w = rng.normal(size=(D, H * hd))
    y = out_projection(o, w)
    ref = F.linear(torch.tensor(o).transpose(1, 2).contiguous().view(B, T, H * hd), torch.tensor(w))
    assert y.shape == (B, T, D) and np.abs(y - ref.numpy()).max() <= 1e-12


def test_out_projection_identity_merges_heads():
    """W_o = I: y[b, t, h*hd + d] is o[b, h, t, d], read with explicit indices."""
    B, H, T, hd = 2, 3, 4, 2
    o = np.random.default_rng(8).normal(size=(B, H, T, hd))
    y = out_projection(o, np.eye(H * hd))
    for b in range(B):
        for h in range(H):
            for t in range(T):
                for d in range(hd):
                    assert y[b, t, h * hd + d] == o[b, h, t, d]


def test_block_matches_torch_sdpa():
    """The whole block of the page (projection, RoPE, causal GQA attention, output projection)
    against torch: F.linear, complex RoPE, repeat_interleave of K/V heads and
    F.scaled_dot_product_attention, all in fp64 (the page's test_against_reference)."""
    B, T, H, KV, hd = 2, 6, 4, 2, 8
    D = H * hd
    x, w = _case(9, B, T, H, KV, hd)
    w_o = np.random.default_rng(10).normal(size=(D, H * hd)) / math.sqrt(D)
    q, k, v = qkv_projection(x, w, H=H, KV=KV, hd=hd, rope_base=10000.0)
    out, _ = attention_prefill(q, k, v, rope_base=0.0, causal=True)
    y = out_projection(out, w_o)

    xt, wt = torch.tensor(x), torch.tensor(w)
    tq = F.linear(xt, wt[:H * hd]).view(B, T, H, hd).transpose(1, 2)
    tk = F.linear(xt, wt[H * hd:(H + KV) * hd]).view(B, T, KV, hd).transpose(1, 2)
    tv = F.linear(xt, wt[(H + KV) * hd:]).view(B, T, KV, hd).transpose(1, 2)
    pos = np.arange(T)
    tq, tk = _torch_rope_complex(tq, pos, 10000.0), _torch_rope_complex(tk, pos, 10000.0)
    g = H // KV
    tk, tv = tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1)
    to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    ty = F.linear(to.transpose(1, 2).contiguous().view(B, T, H * hd), torch.tensor(w_o))
    assert np.abs(y - ty.numpy()).max() <= 1e-12
