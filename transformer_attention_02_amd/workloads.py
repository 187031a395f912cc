"""Seeded synthetic inputs and the workload table.

This module draws random numbers and nothing else: it holds none of the
attention arithmetic (no rotation, no softmax, no masking), so the HIP path and
the CPU oracle can both be fed from it without sharing any of the method.

Every tensor is produced on the host from a fixed seed:

* the tiny fp32 case is the seeded instance of the "Write attention from
  scratch" lab page (NumPy ``default_rng(0)``; draws x, Wq, Wk, Wv, Wo in that
  order, weights scaled by 1/sqrt(d)); its Q/K/V are ``x @ W`` in fp64, split
  into heads and stored as fp32;
* the bf16 cases draw fp32 N(0,1) from ``torch.Generator().manual_seed(seed)``
  in the order q, k, v and round each value to bf16 (round to nearest even);
* the decode case draws context lengths with NumPy ``default_rng(5)``
  (integers in [512, 8192], both ends inclusive), then q, k_new, v_new and the
  valid prefix of each sequence's K/V cache from a torch generator; cache rows
  at or past a sequence's length are zero and are never read.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    T: int
    H: int
    KV: int
    hd: int
    dtype: str
    seed: int
    rope_base: float  # 0.0 means no rotary embedding
    pos0: int = 0
    causal: bool = True
    alibi: int = 0  # 0 none, 1 geometric 2^(-8(h+1)/H), 2 page-1 heuristic 2^(-2(h+1)/H)
    Tq: int = 0        # query rows (a chunk of the T tokens); 0 means all T
    q_offset: int = 0  # token index of the first query row
    window: int = 0    # sliding window in tokens (causal only); 0 means none

    @property
    def rows(self) -> int:
        return self.Tq or self.T

    def pairs(self) -> int:
        """Visible (query, key) pairs per head: causal keys up to the query's own
        token, within the window if any; all T keys when not causal."""
        if not self.causal:
            return self.rows * self.T
        if not self.window:
            a, b = self.q_offset + 1, self.q_offset + self.rows   # sum of (t + 1) over the chunk
            return (a + b) * self.rows // 2
        return sum(min(t + 1, self.window) for t in range(self.q_offset, self.q_offset + self.rows))

    def flops(self) -> float:
        """Algorithmic flops: two contractions over the visible (query, key) pairs."""
        return 4.0 * self.B * self.H * self.hd * self.pairs()

    def bwd_flops(self) -> float:
        """Algorithmic flops of the backward: five contractions over the visible
        pairs (the scores again, dP, dV, dK and dQ), 2.5 times the forward."""
        return 10.0 * self.B * self.H * self.hd * self.pairs()

    def io_bytes(self, out_elem: int = 4) -> int:
        e = 4 if self.dtype == F32 else 2
        return (self.B * self.H * self.T * self.hd * (e + out_elem)
                + 2 * self.B * self.KV * self.T * self.hd * e)


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H: int
    KV: int
    hd: int
    len_lo: int
    len_hi: int
    len_seed: int
    seed: int
    rope_base: float
    alibi: int = 0
    dtype: str = BF16
    cache: str = "same"    # "same": the cache has dtype; "fp8": OCP E4M3 codes with k_scale / v_scale
    k_scale: float = 1.0
    v_scale: float = 1.0

    def lengths(self) -> np.ndarray:
        rng = np.random.default_rng(self.len_seed)
        return rng.integers(self.len_lo, self.len_hi, size=self.B, endpoint=True).astype(np.int32)

    def lmax(self) -> int:
        return int(self.lengths().max()) + 1

    def kv_read_bytes(self) -> int:
        """K and V bytes the step must read: (len_b + 1) rows of K and V per KV head."""
        e = 1 if self.cache == "fp8" else (4 if self.dtype == F32 else 2)
        return int(sum(int(L) + 1 for L in self.lengths()) * self.KV * self.hd * 2 * e)


@dataclass(frozen=True)
class LatentDecodeWorkload:
    """Decode over a latent cache: one dc-dim latent per token shared by H heads,
    per-head up-projections W_uk / W_uv [H, dc, hd] (bf16)."""
    name: str
    B: int
    H: int
    hd: int
    dc: int
    len_lo: int
    len_hi: int
    len_seed: int
    seed: int
    alibi: int = 0

    def lengths(self) -> np.ndarray:
        rng = np.random.default_rng(self.len_seed)
        return rng.integers(self.len_lo, self.len_hi, size=self.B, endpoint=True).astype(np.int32)

    def cache_read_bytes(self) -> int:
        """Latent bytes the step must read: (len_b + 1) rows of dc bf16 per sequence."""
        return int(sum(int(L) + 1 for L in self.lengths()) * self.dc * 2)


@dataclass(frozen=True)
class ProjWorkload:
    """The projections either side of attention: x [B, T, D] -> q/k/v heads
    (w_qkv [(H+2KV)hd, D]) and the attention output [B, H, T, hd] -> y [B, T, D]
    (w_o [D, H hd]); bf16."""
    name: str
    B: int
    T: int
    D: int
    H: int
    KV: int
    hd: int
    rope_base: float
    seed: int

    @property
    def M(self) -> int:
        return self.B * self.T

    @property
    def N_qkv(self) -> int:
        return (self.H + 2 * self.KV) * self.hd

    def qkv_flops(self) -> float:
        return 2.0 * self.M * self.N_qkv * self.D

    def out_flops(self) -> float:
        return 2.0 * self.M * self.D * self.H * self.hd


TINY_FP32 = PrefillWorkload("tiny-fp32 T=6 H=4 KV=2 hd=8", 1, 6, 4, 2, 8, F32, 0, 10000.0)
SMALL_BF16 = PrefillWorkload("small-bf16 B=1 T=512 H=8 KV=2 hd=64", 1, 512, 8, 2, 64, BF16, 2, 10000.0)
LLAMA3_8B = PrefillWorkload("llama3-8b-prefill B=4 T=4096 H=32 KV=8 hd=128 rope=5e5",
                            4, 4096, 32, 8, 128, BF16, 3, 500000.0)
ALIBI_MHA = PrefillWorkload("alibi-mha-prefill B=8 T=2048 H=16 KV=16 hd=128",
                            8, 2048, 16, 16, 128, BF16, 4, 0.0, alibi=1)
# the Llama-3-8B prompt with a 1024-token sliding window, and its last 512
# tokens processed as one chunk against the whole prompt's keys (same inputs)
LLAMA3_WINDOW = PrefillWorkload("llama3-8b-prefill sliding window W=1024 B=4 T=4096 H=32 KV=8 hd=128 rope=5e5",
                                4, 4096, 32, 8, 128, BF16, 3, 500000.0, window=1024)
LLAMA3_CHUNK = PrefillWorkload("llama3-8b chunked prefill: tokens 3584..4095 over 4096 keys, B=4 H=32 KV=8 hd=128",
                               4, 4096, 32, 8, 128, BF16, 3, 500000.0, Tq=512, q_offset=3584)
KV_DECODE = DecodeWorkload("kv-decode B=64 len~U[512,8192] H=32 KV=8 hd=128",
                           64, 32, 8, 128, 512, 8192, 5, 5, 10000.0)
# the same step over an fp8 cache: the bf16 draws above, stored as E4M3 codes of
# value * 64 (|N(0,1)| * 64 stays well inside the +-448 range)
KV_DECODE_FP8 = DecodeWorkload("kv-decode fp8 E4M3 cache (scale 1/64) B=64 len~U[512,8192] H=32 KV=8 hd=128",
                               64, 32, 8, 128, 512, 8192, 5, 5, 10000.0, cache="fp8", k_scale=1 / 64,
                               v_scale=1 / 64)

# latent-cache decode over the same 64 sequence lengths: 16 heads of 128 dims
# up-projected from 512-number latents (the cache holds 1 KiB per token)
LATENT_DECODE = LatentDecodeWorkload("latent-decode B=64 len~U[512,8192] H=16 hd=128 dc=512",
                                     64, 16, 128, 512, 512, 8192, 5, 6)

# the projections of the Llama-3-8B prefill shape: D = 4096 = 32 x 128, 8 KV heads
PROJ_LLAMA3_8B = ProjWorkload("llama3-8b projections B=4 T=4096 D=4096 H=32 KV=8 hd=128 rope=5e5",
                              4, 4096, 4096, 32, 8, 128, 500000.0, 7)

PREFILL_WORKLOADS = {"tiny": TINY_FP32, "small": SMALL_BF16, "llama3": LLAMA3_8B, "alibi": ALIBI_MHA,
                     "window": LLAMA3_WINDOW, "chunk": LLAMA3_CHUNK}


def lab_instance():
    """The seeded instance of the attention lab page: x, Wq, Wk, Wv, Wo (fp64).

    T=6 tokens, width d=32, H=4 query heads, KV=2 key/value heads, hd=8.
    """
    T, d, H, KV = 6, 32, 4, 2
    hd = d // H
    # One generator seeded with 0 draws, in order, the tokens x (unscaled) and the
    # query, key, value and output weights, each divided by sqrt(d): the page's
    # draw order, which its two printed checks depend on.
    draws = (((T, d), 1.0), ((d, H * hd), np.sqrt(d)), ((d, KV * hd), np.sqrt(d)), ((d, KV * hd), np.sqrt(d)),
             ((H * hd, d), np.sqrt(d)))
    rng = np.random.default_rng(0)
    return tuple(rng.normal(size=shape) / div for shape, div in draws)


def split_heads(y: np.ndarray, heads: int) -> np.ndarray:
    """[T, heads*hd] -> [1, heads, T, hd] (a reshape; no arithmetic)."""
    T = y.shape[0]
    return np.ascontiguousarray(y.reshape(T, heads, -1).transpose(1, 0, 2)[None])


def tiny_qkv(x: np.ndarray | None = None):
    """Q/K/V of the lab instance as fp32 arrays [1,H,T,hd], [1,KV,T,hd] (host projections)."""
    x0, Wq, Wk, Wv, _ = lab_instance()
    if x is None:
        x = x0
    q = split_heads(x @ Wq, 4).astype(np.float32)
    k = split_heads(x @ Wk, 2).astype(np.float32)
    v = split_heads(x @ Wv, 2).astype(np.float32)
    return q, k, v


def normal_bf16(gen: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def normal_f32(gen: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32)


def prefill_inputs(w: PrefillWorkload, *, B: int | None = None, T: int | None = None):
    """Host tensors q [B,H,T,hd], k, v [B,KV,T,hd] for a prefill workload.

    ``B``/``T`` override the sizes (same seed and draw order) for scaled-down cases.
    """
    B = w.B if B is None else B
    T = w.T if T is None else T
    if w is TINY_FP32 and B == 1 and T == 6:
        q, k, v = tiny_qkv()
        return torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)
    g = torch.Generator().manual_seed(w.seed)
    draw = normal_bf16 if w.dtype == BF16 else normal_f32
    q = draw(g, (B, w.H, T, w.hd))
    k = draw(g, (B, w.KV, T, w.hd))
    v = draw(g, (B, w.KV, T, w.hd))
    if w.Tq:  # a chunk: the query rows of those tokens, drawn with the whole prompt
        q = q[:, :, w.q_offset:w.q_offset + w.Tq].contiguous()
    return q, k, v


def prefill_dout(w: PrefillWorkload, *, B: int | None = None, T: int | None = None):
    """Host tensor dout [B,H,rows,hd]: the upstream gradient for a backward
    step, N(0,1) rounded like the inputs, from its own seed (w.seed + 1000)."""
    B = w.B if B is None else B
    T = w.rows if T is None else T
    g = torch.Generator().manual_seed(w.seed + 1000)
    draw = normal_bf16 if w.dtype == BF16 else normal_f32
    return draw(g, (B, w.H, T, w.hd))


def random_prefill(seed: int, B: int, T: int, H: int, KV: int, hd: int, dtype: str = BF16, scale: float = 1.0):
    """Generic seeded q/k/v for parity sweeps (same draw order as the workloads)."""
    g = torch.Generator().manual_seed(seed)
    draw = normal_bf16 if dtype == BF16 else normal_f32
    q = draw(g, (B, H, T, hd))
    k = draw(g, (B, KV, T, hd))
    v = draw(g, (B, KV, T, hd))
    if scale != 1.0:
        q = (q.float() * scale).to(q.dtype)
        k = (k.float() * scale).to(k.dtype)
    return q, k, v


@dataclass
class DecodeInputs:
    q: torch.Tensor        # [B, H, hd]
    k_new: torch.Tensor    # [B, KV, hd]
    v_new: torch.Tensor    # [B, KV, hd]
    k_cache: torch.Tensor  # [B, KV, Lmax, hd] (valid prefix per sequence; rest zero)
    v_cache: torch.Tensor
    lens: np.ndarray       # [B] int32
    extra: dict = field(default_factory=dict)


def decode_inputs(w: DecodeWorkload, *, B: int | None = None, lens: np.ndarray | None = None,
                  lmax: int | None = None, device: str | torch.device = "cpu") -> DecodeInputs:
    """Seeded decode inputs. The cache is filled sequence by sequence (draw order b = 0..B-1)
    directly into a tensor on ``device`` so that the full-size cache never exists twice."""
    if lens is None:
        lens = w.lengths()
    lens = np.asarray(lens, dtype=np.int32)
    if B is not None:
        lens = lens[:B]
    B = len(lens)
    Lmax = int(lens.max()) + 1 if lmax is None else lmax
    g = torch.Generator().manual_seed(w.seed)
    draw = normal_bf16 if w.dtype == BF16 else normal_f32
    q = draw(g, (B, w.H, w.hd))
    k_new = draw(g, (B, w.KV, w.hd))
    v_new = draw(g, (B, w.KV, w.hd))
    tdt = torch.bfloat16 if w.dtype == BF16 else torch.float32
    k_cache = torch.zeros(B, w.KV, Lmax, w.hd, dtype=tdt, device=device)
    v_cache = torch.zeros(B, w.KV, Lmax, w.hd, dtype=tdt, device=device)
    if w.cache == "fp8":
        k_cache = torch.zeros(B, w.KV, Lmax, w.hd, dtype=torch.uint8, device=device)
        v_cache = torch.zeros(B, w.KV, Lmax, w.hd, dtype=torch.uint8, device=device)
    for b in range(B):
        L = int(lens[b])
        kx = draw(g, (w.KV, L, w.hd))
        vx = draw(g, (w.KV, L, w.hd))
        if w.cache == "fp8":
            kx, vx = to_e4m3_codes(kx, w.k_scale), to_e4m3_codes(vx, w.v_scale)
        k_cache[b, :, :L] = kx.to(device)
        v_cache[b, :, :L] = vx.to(device)
    return DecodeInputs(q, k_new, v_new, k_cache, v_cache, lens)


def to_e4m3_codes(x: torch.Tensor, scale: float) -> torch.Tensor:
    """uint8 OCP E4M3 codes of x / scale by torch's own float8_e4m3fn conversion
    (round to nearest even), clamped to the finite range first; used only to
    synthesise fp8 cache contents."""
    return (x.float() / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


@dataclass
class LatentInputs:
    q: torch.Tensor        # [B, H, hd]
    c_new: torch.Tensor    # [B, dc]
    c_cache: torch.Tensor  # [B, Lmax, dc] (valid prefix per sequence; rest zero)
    w_uk: torch.Tensor     # [H, dc, hd]
    w_uv: torch.Tensor     # [H, dc, hd]
    lens: np.ndarray       # [B]


def latent_decode_inputs(w: LatentDecodeWorkload, *, lens: np.ndarray | None = None, lmax: int | None = None,
                         device: str | torch.device = "cpu") -> LatentInputs:
    """Seeded bf16 inputs: q, c_new, W_uk, W_uv (N(0,1), the weights scaled by
    1/sqrt(dc) before rounding), then each sequence's latent prefix."""
    if lens is None:
        lens = w.lengths()
    lens = np.asarray(lens, dtype=np.int32)
    B = len(lens)
    Lmax = int(lens.max()) + 1 if lmax is None else lmax
    g = torch.Generator().manual_seed(w.seed)
    q = normal_bf16(g, (B, w.H, w.hd))
    c_new = normal_bf16(g, (B, w.dc))
    w_uk = (torch.randn(w.H, w.dc, w.hd, generator=g) / np.sqrt(w.dc)).to(torch.bfloat16)
    w_uv = (torch.randn(w.H, w.dc, w.hd, generator=g) / np.sqrt(w.dc)).to(torch.bfloat16)
    c_cache = torch.zeros(B, Lmax, w.dc, dtype=torch.bfloat16, device=device)
    for b in range(B):
        L = int(lens[b])
        c_cache[b, :L] = normal_bf16(g, (L, w.dc)).to(device)
    return LatentInputs(q, c_new, c_cache, w_uk, w_uv, lens)


@dataclass
class ProjInputs:
    x: torch.Tensor      # [B, T, D]
    w_qkv: torch.Tensor  # [(H + 2KV) hd, D]
    o: torch.Tensor      # [B, H, T, hd], an attention output to project back
    w_o: torch.Tensor    # [D, H hd]


def proj_inputs(w: ProjWorkload, *, B: int | None = None, T: int | None = None) -> ProjInputs:
    """Seeded bf16 inputs: x and o N(0,1); weights N(0,1) scaled by 1/sqrt(fan-in)
    before rounding (the scale of nn.Linear's default initialisation)."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    g = torch.Generator().manual_seed(w.seed)
    x = normal_bf16(g, (B, T, w.D))
    w_qkv = (torch.randn(w.N_qkv, w.D, generator=g) / np.sqrt(w.D)).to(torch.bfloat16)
    o = normal_bf16(g, (B, w.H, T, w.hd))
    w_o = (torch.randn(w.D, w.H * w.hd, generator=g) / np.sqrt(w.H * w.hd)).to(torch.bfloat16)
    return ProjInputs(x, w_qkv, o, w_o)
