"""HIP graph capture of the library's entry points, through the C ABI.

An entry point only launches kernels on the caller's stream. It does not
allocate, free, memset or synchronise, so a whole step can be recorded into a
HIP graph (torch.cuda.CUDAGraph over hipStreamBeginCapture) and replayed.

Each graph below holds a chain of calls. Every replay must reproduce the eager
results bitwise. Between replays the outputs are overwritten with NaN by an
eager fill kernel, and unrelated eager work runs. A replay that skipped a kernel,
read stale scratch memory or depended on state left by an earlier call would
therefore fail.
"""
import numpy as np
import pytest
import torch

from transformer_attention_02_amd import binding as bd
from transformer_attention_02_amd import workloads as W

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _replay_and_compare(step, what):
    """Run `step` eagerly (reference), capture it, then replay REPLAYS times."""
    ref = {k: t.clone() for k, t in step().items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capturing stream's side, as torch recommends
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    g = torch.Generator(device="cuda").manual_seed(3)
    for r in range(REPLAYS):
        print(f"[graph] {what} replay {r}", flush=True)
        for t in outs.values():
            t.fill_(float("nan"))
        a = torch.randn(1024, 1024, device="cuda", generator=g)
        (a @ a).sum().item()  # unrelated eager work, with a synchronisation
        graph.replay()
        torch.cuda.synchronize()
        for k, t in outs.items():
            assert torch.isfinite(t.float()).all(), f"{what}: replay {r} left {k} unwritten"
            assert torch.equal(t, ref[k]), f"{what}: replay {r} differs from the eager {k}"


def test_graph_attention_block():
    """QKV projection with RoPE -> causal attention (rotation off) -> output projection."""
    B, T, D, H, KV, hd = 2, 300, 256, 4, 2, 64
    g = torch.Generator().manual_seed(97)
    x = W.normal_bf16(g, (B, T, D)).cuda()
    w_qkv = (torch.randn((H + 2 * KV) * hd, D, generator=g) / np.sqrt(D)).to(torch.bfloat16).cuda()
    w_o = (torch.randn(D, H * hd, generator=g) / np.sqrt(H * hd)).to(torch.bfloat16).cuda()

    def step():
        q, k, v = bd.qkv_proj(x, w_qkv, H, KV, rope_base=10000.0)
        o, lse = bd.prefill(q, k, v, rope_base=0.0, causal=True, out_dtype=torch.bfloat16)
        y = bd.out_proj(o, w_o, out_dtype=torch.float32)
        return {"q": q, "k": k, "v": v, "o": o, "lse": lse, "y": y}

    _replay_and_compare(step, "block")


def test_graph_prefill_with_rotation_and_backward():
    """The rotated-K pre-pass, the forward and the backward (rotated copies, D, dq and dk/dv kernels),
    with their workspaces allocated before capture."""
    B, T, H, KV, hd = 2, 333, 8, 2, 128
    q, k, v = (t.cuda() for t in W.random_prefill(98, B, T, H, KV, hd))
    g = torch.Generator().manual_seed(99)
    dout = W.normal_bf16(g, (B, H, T, hd)).cuda()
    ws, _ = bd.prefill_workspace(B, T, KV, hd, bd.ATTN_DTYPE_BF16, 10000.0, "cuda")
    nb = bd.attn_prefill_bwd_workspace_bytes(B, T, H, KV, hd, bd.ATTN_DTYPE_BF16, 10000.0)
    bws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")

    def step():
        out, lse = bd.prefill(q, k, v, rope_base=10000.0, causal=True, out_dtype=torch.bfloat16, workspace=ws)
        dq, dk, dv = bd.prefill_bwd(q, k, v, out, lse, dout, rope_base=10000.0, causal=True,
                                    grad_dtype=torch.bfloat16, workspace=bws)
        return {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}

    _replay_and_compare(step, "prefill+backward")


def test_graph_decode_steps():
    """One decode step of each kind: bf16 cache with append, the projection writing the cache
    followed by the decode without append, fp8 cache, latent cache. Replays append the same token
    to the same slot, so every replay sees the same inputs."""
    lens = np.array([0, 1, 255, 700, 1500, 3000], dtype=np.int32)
    w16 = W.DecodeWorkload("graph-decode", 6, 8, 2, 128, 0, 0, 5, 111, 10000.0)
    d16 = W.decode_inputs(w16, lens=lens, lmax=3001, device="cuda")
    w8 = W.DecodeWorkload("graph-decode-fp8", 6, 8, 2, 128, 0, 0, 5, 112, 10000.0, cache="fp8",
                          k_scale=1 / 64, v_scale=1 / 64)
    d8 = W.decode_inputs(w8, lens=lens, lmax=3001, device="cuda")
    wl = W.LatentDecodeWorkload("graph-latent", 6, 16, 128, 512, 0, 0, 5, 113)
    dl = W.latent_decode_inputs(wl, lens=lens, lmax=3001, device="cuda")
    lens_d = torch.from_numpy(lens).cuda()
    g = torch.Generator().manual_seed(114)
    B, H, KV, hd, D = 6, 8, 2, 128, 512
    x = W.normal_bf16(g, (B, 1, D)).cuda()
    w_qkv = (torch.randn((H + 2 * KV) * hd, D, generator=g) / np.sqrt(D)).to(torch.bfloat16).cuda()
    kc2 = torch.zeros_like(d16.k_cache)
    vc2 = torch.zeros_like(d16.v_cache)
    kc2[:, :, :3000] = d16.k_cache[:, :, :3000]
    vc2[:, :, :3000] = d16.v_cache[:, :, :3000]
    ws16, _ = bd.decode_workspace(B, H, KV, hd, 3001, "cuda")
    ws16b, _ = bd.decode_workspace(B, H, KV, hd, 3001, "cuda")
    ws8, _ = bd.decode_workspace(B, H, KV, hd, 3001, "cuda")
    nl = bd.attn_decode_latent_workspace_bytes(B, 16, 512, 3001)
    wsl = torch.empty(max(nl, 1), dtype=torch.uint8, device="cuda")
    qd, knd, vnd = d16.q.cuda(), d16.k_new.cuda(), d16.v_new.cuda()
    q8, kn8, vn8 = d8.q.cuda(), d8.k_new.cuda(), d8.v_new.cuda()
    ql, cnl, wuk, wuv = dl.q.cuda(), dl.c_new.cuda(), dl.w_uk.cuda(), dl.w_uv.cuda()

    def step():
        o1, l1 = bd.decode(qd, knd, vnd, d16.k_cache, d16.v_cache, lens_d, rope_base=10000.0,
                           out_dtype=torch.float32, workspace=ws16)
        qp = bd.qkv_proj_cache(x, w_qkv, kc2, vc2, lens_d, H, rope_base=10000.0)
        o2, l2 = bd.decode(qp[:, :, 0].contiguous(), None, None, kc2, vc2, lens_d, rope_base=0.0,
                           out_dtype=torch.float32, workspace=ws16b)
        o3, l3 = bd.decode_fp8(q8, kn8, vn8, d8.k_cache, d8.v_cache, lens_d, 1 / 64, 1 / 64, rope_base=10000.0,
                               out_dtype=torch.float32, workspace=ws8)
        o4, l4 = bd.decode_latent(ql, cnl, dl.c_cache, lens_d, wuk, wuv, out_dtype=torch.float32, workspace=wsl)
        return {"o1": o1, "l1": l1, "qp": qp, "o2": o2, "l2": l2, "o3": o3, "l3": l3, "o4": o4, "l4": l4}

    _replay_and_compare(step, "decode")


def test_graph_wave_split_prefill(monkeypatch):
    """The small prefill's shape with the wave-split workgroups forced: the rotated-K pre-pass, then the kernel
    whose four waves each walk a share of a block's key tiles and merge through LDS."""
    monkeypatch.delenv("ATTN_PREFILL_WAVES", raising=False)
    monkeypatch.setenv("ATTN_PREFILL_WSPLIT", "1")
    w = W.SMALL_BF16
    q, k, v = (t.cuda() for t in W.prefill_inputs(w))
    ws, _ = bd.prefill_workspace(w.B, w.T, w.KV, w.hd, bd.ATTN_DTYPE_BF16, w.rope_base, "cuda")

    def step():
        o, lse = bd.prefill(q, k, v, rope_base=w.rope_base, out_dtype=torch.bfloat16, workspace=ws)
        return {"o": o, "lse": lse}

    _replay_and_compare(step, "wave-split prefill")
