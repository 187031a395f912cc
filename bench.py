#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  1. prefill: causal GQA + RoPE attention forward, Llama-3-8B shape
     (B=4, T=4096, H=32, KV=8, hd=128, RoPE base 5e5, bf16 in, bf16 out);
  2. decode: one KV-cache decode step for 64 sequences with context lengths
     drawn uniformly from [512, 8192] (H=32, KV=8, hd=128, RoPE base 1e4).

Prints ONE JSON line. ``value`` is prefill TFLOP/s (algorithmic flops
4*B*H*hd*T(T+1)/2 over the time of the prefill call); the decode KV-read GB/s
(sum over sequences of (len+1)*KV*hd*2*2 bytes over the time of the decode
call) is in ``decode``. ``roofline`` is for the dominant kernel (the prefill
attention kernel), timed with HIP events that the library records around that
kernel on its own stream; ``decode.roofline`` is the same for the split-KV
kernel. ``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the
same workload.

``--workload decode-fp8`` times attn_decode_fp8_fwd on the same decode step over
an fp8 (OCP E4M3) cache, with the bf16-cache step in the same run for the
before/after comparison; ``value`` = fp8 KV bytes read per second.

``--workload latent-decode`` times attn_decode_latent_fwd: 64 sequences of the
same lengths over a cache of one 512-number latent per token (16 heads of 128
dims up-projected from it); ``value`` = latent bytes read per second.

``--workload backward`` times attn_prefill_bwd on the Llama-3-8B prefill
instead (bf16 gradients; ``value`` = backward TFLOP/s with the algorithmic
10*B*H*hd*T(T+1)/2 flops; ``roofline`` covers its two matrix-core kernels,
dq and dk/dv, timed together).

``--workload proj`` times the projections either side of attention on the
Llama-3-8B prefill shape (B=4, T=4096, D=4096, H=32, KV=8, hd=128):
attn_qkv_proj_fwd (fused QKV projection, RoPE of q and k, head split) then
attn_out_proj_fwd (head merge, output projection); ``value`` = TFLOP/s of the
pair, ``roofline`` covers the QKV kernel, and the same two GEMMs through
torch.matmul (the vendor library, without the epilogue work) are timed in the
same run as context.

``--workload block`` times the whole attention block of that page's module on
the Llama-3-8B shape: the QKV projection with RoPE, causal GQA attention (the
rotation off: q and k arrive rotated) and the output projection; ``value`` =
TFLOP/s of the block (projections + attention), tokens per second in
``config``, ``roofline`` for the block's longest kernel.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workload all|prefill|decode|decode-fp8|latent-decode|proj|block|alibi|small|window|chunk|backward|copy]
                       [--no-cpu-baseline] [--no-ceilings]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal GQA+RoPE attn fwd TFLOP/s (prefill) + KV-read GB/s (decode), 1 GPU"
# MI355X: 256 CUs x 4096 dense bf16 flop/clk/CU x 2.4 GHz; HBM3E 8 TB/s.
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded (same SONAME)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventCreate.restype = ctypes.c_int
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.restype = ctypes.c_int
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self):
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.made.append(ev.value)
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(e)
        self.made = []


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, sources, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source and this workload (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            tab = json.load(f)
    except (OSError, ValueError):
        return None
    ent = tab.get(f"{kernel} @ {workload}")
    if not ent or ent.get("source_digest") != source_digest(sources) or ent.get("workload") != workload:
        return None
    return ent.get("bytes_per_launch")


PROJ_SOURCES = ["transformer_attention_02_amd/csrc/proj.hip", "transformer_attention_02_amd/csrc/proj_internal.h",
                "transformer_attention_02_amd/csrc/mfma_tile.h", "transformer_attention_02_amd/csrc/attn_internal.h"]
PREFILL_SOURCES = ["transformer_attention_02_amd/csrc/prefill_mfma.hip", "transformer_attention_02_amd/csrc/mfma_tile.h",
                   "transformer_attention_02_amd/csrc/attn_internal.h"]
LATENT_SOURCES = ["transformer_attention_02_amd/csrc/decode_latent.hip", "transformer_attention_02_amd/csrc/mfma_tile.h",
                  "transformer_attention_02_amd/csrc/attn_internal.h"]
BACKWARD_SOURCES = ["transformer_attention_02_amd/csrc/backward_mfma.hip", "transformer_attention_02_amd/csrc/mfma_tile.h",
                    "transformer_attention_02_amd/csrc/attn_internal.h"]
DECODE_SOURCES = ["transformer_attention_02_amd/csrc/decode.hip", "transformer_attention_02_amd/csrc/attn_internal.h"]


class Prefill:
    def __init__(self, w, dev, bd, W, torch):
        self.w, self.bd = w, bd
        q, k, v = W.prefill_inputs(w)
        self.q, self.k, self.v = q.to(dev), k.to(dev), v.to(dev)
        self.out = torch.empty(w.B, w.H, w.rows, w.hd, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(w.B, w.H, w.rows, dtype=torch.float32, device=dev)
        dt = bd.ATTN_DTYPE_BF16 if w.dtype == "bf16" else bd.ATTN_DTYPE_F32
        self.dt = dt
        self.ws, self.ws_bytes = bd.prefill_workspace(w.B, w.T, w.KV, w.hd, dt, w.rope_base, dev)

    def __call__(self, stream, events=None):
        w, bd = self.w, self.bd
        if events:
            bd.attn_set_timing_events(*events)
        if w.Tq or w.q_offset or w.window:
            st = bd.attn_prefill_ex_fwd(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.out.data_ptr(),
                                        self.lse.data_ptr(), w.B, w.rows, w.T, w.H, w.KV, w.hd, w.pos0, w.q_offset,
                                        w.window, w.rope_base, int(w.causal), w.alibi, self.dt, bd.ATTN_DTYPE_BF16,
                                        self.ws.data_ptr(), self.ws_bytes, stream)
        else:
            st = bd.attn_prefill_fwd(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.out.data_ptr(),
                                     self.lse.data_ptr(), w.B, w.T, w.H, w.KV, w.hd, w.pos0, w.rope_base,
                                     int(w.causal), w.alibi, self.dt, bd.ATTN_DTYPE_BF16, self.ws.data_ptr(),
                                     self.ws_bytes, stream)
        if st != bd.ATTN_OK:
            raise RuntimeError(f"attn_prefill_fwd: {bd.attn_status_str(st)} {bd.attn_last_error()}")

    def work(self):
        return self.w.flops()


class Decode:
    def __init__(self, w, dev, bd, W, torch):
        self.w, self.bd = w, bd
        inp = W.decode_inputs(w, device=dev)
        self.inp = inp
        self.q, self.kn, self.vn = inp.q.to(dev), inp.k_new.to(dev), inp.v_new.to(dev)
        self.kc, self.vc = inp.k_cache, inp.v_cache
        self.lens = torch.from_numpy(inp.lens).to(dev)
        self.Lmax = self.kc.shape[2]
        self.out = torch.empty(inp.q.shape, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(inp.q.shape[:2], dtype=torch.float32, device=dev)
        self.ws, self.ws_bytes = bd.decode_workspace(w.B, w.H, w.KV, w.hd, self.Lmax, dev)

    def __call__(self, stream, events=None):
        w, bd = self.w, self.bd
        if events:
            bd.attn_set_timing_events(*events)
        st = bd.attn_decode_fwd(self.q.data_ptr(), self.kn.data_ptr(), self.vn.data_ptr(), self.kc.data_ptr(),
                                self.vc.data_ptr(), self.lens.data_ptr(), self.out.data_ptr(), self.lse.data_ptr(),
                                w.B, w.H, w.KV, w.hd, self.Lmax, w.rope_base, w.alibi, bd.ATTN_DTYPE_BF16,
                                bd.ATTN_DTYPE_BF16, self.ws.data_ptr(), self.ws_bytes, stream)
        if st != bd.ATTN_OK:
            raise RuntimeError(f"attn_decode_fwd: {bd.attn_status_str(st)} {bd.attn_last_error()}")

    def work(self):
        return self.w.kv_read_bytes()


class DecodeFp8(Decode):
    """attn_decode_fp8_fwd over uint8 E4M3 caches (same shapes as Decode)."""

    def __call__(self, stream, events=None):
        w, bd = self.w, self.bd
        if events:
            bd.attn_set_timing_events(*events)
        st = bd.attn_decode_fp8_fwd(self.q.data_ptr(), self.kn.data_ptr(), self.vn.data_ptr(), self.kc.data_ptr(),
                                    self.vc.data_ptr(), self.lens.data_ptr(), self.out.data_ptr(),
                                    self.lse.data_ptr(), w.B, w.H, w.KV, w.hd, self.Lmax, w.rope_base, w.alibi,
                                    w.k_scale, w.v_scale, bd.ATTN_DTYPE_BF16, bd.ATTN_DTYPE_BF16, self.ws.data_ptr(),
                                    self.ws_bytes, stream)
        if st != bd.ATTN_OK:
            raise RuntimeError(f"attn_decode_fp8_fwd: {bd.attn_status_str(st)} {bd.attn_last_error()}")


class LatentDecode:
    """attn_decode_latent_fwd on the latent-cache workload (inputs resident on the GPU)."""

    def __init__(self, w, dev, bd, W, torch):
        self.w, self.bd = w, bd
        inp = W.latent_decode_inputs(w, device=dev)
        self.inp = inp
        self.q, self.cn = inp.q.to(dev), inp.c_new.to(dev)
        self.wk, self.wv = inp.w_uk.to(dev), inp.w_uv.to(dev)
        self.cc = inp.c_cache
        self.lens = torch.from_numpy(inp.lens).to(dev)
        self.Lmax = self.cc.shape[1]
        self.out = torch.empty(w.B, w.H, w.hd, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(w.B, w.H, dtype=torch.float32, device=dev)
        self.ws_bytes = bd.attn_decode_latent_workspace_bytes(w.B, w.H, w.dc, self.Lmax)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev)

    def __call__(self, stream, events=None):
        w, bd = self.w, self.bd
        if events:
            bd.attn_set_timing_events(*events)
        st = bd.attn_decode_latent_fwd(self.q.data_ptr(), self.cn.data_ptr(), self.cc.data_ptr(), self.lens.data_ptr(),
                                       self.wk.data_ptr(), self.wv.data_ptr(), self.out.data_ptr(),
                                       self.lse.data_ptr(), w.B, w.H, w.hd, w.dc, self.Lmax, w.alibi,
                                       bd.ATTN_DTYPE_BF16, bd.ATTN_DTYPE_BF16, self.ws.data_ptr(), self.ws_bytes,
                                       stream)
        if st != bd.ATTN_OK:
            raise RuntimeError(f"attn_decode_latent_fwd: {bd.attn_status_str(st)} {bd.attn_last_error()}")


class Proj:
    """attn_qkv_proj_fwd then attn_out_proj_fwd (inputs resident on the GPU); each kernel timed."""

    def __init__(self, w, dev, bd, W, torch):
        self.w, self.bd = w, bd
        inp = W.proj_inputs(w)
        self.x, self.wq = inp.x.to(dev), inp.w_qkv.to(dev)
        self.o, self.wo = inp.o.to(dev), inp.w_o.to(dev)
        bf = torch.bfloat16
        self.q = torch.empty(w.B, w.H, w.T, w.hd, dtype=bf, device=dev)
        self.k = torch.empty(w.B, w.KV, w.T, w.hd, dtype=bf, device=dev)
        self.v = torch.empty(w.B, w.KV, w.T, w.hd, dtype=bf, device=dev)
        self.y = torch.empty(w.B, w.T, w.D, dtype=bf, device=dev)

    def __call__(self, stream, ev_qkv=None, ev_out=None):
        w, bd = self.w, self.bd
        if ev_qkv:
            bd.attn_set_timing_events(*ev_qkv)
        st = bd.attn_qkv_proj_fwd(self.x.data_ptr(), self.wq.data_ptr(), self.q.data_ptr(), self.k.data_ptr(),
                                  self.v.data_ptr(), w.B, w.T, w.D, w.H, w.KV, w.hd, 0, w.rope_base,
                                  bd.ATTN_DTYPE_BF16, stream)
        if st != bd.ATTN_OK:
            raise RuntimeError(f"attn_qkv_proj_fwd: {bd.attn_status_str(st)} {bd.attn_last_error()}")
        if ev_out:
            bd.attn_set_timing_events(*ev_out)
        st = bd.attn_out_proj_fwd(self.o.data_ptr(), self.wo.data_ptr(), self.y.data_ptr(), w.B, w.T, w.H, w.hd, w.D,
                                  bd.ATTN_DTYPE_BF16, bd.ATTN_DTYPE_BF16, stream)
        if st != bd.ATTN_OK:
            raise RuntimeError(f"attn_out_proj_fwd: {bd.attn_status_str(st)} {bd.attn_last_error()}")

    def library_gemms(self, torch, reps=10):
        """The same two GEMMs through torch.matmul (no rotation, no head split): ms each."""
        w = self.w
        x2 = self.x.view(w.M, w.D)
        o2 = self.o.transpose(1, 2).contiguous().view(w.M, w.H * w.hd)
        out = {}
        for name, f in (("qkv", lambda: torch.matmul(x2, self.wq.t())), ("out", lambda: torch.matmul(o2, self.wo.t()))):
            for _ in range(3):
                f()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            torch.cuda.synchronize()
            out[name] = e0.elapsed_time(e1) / reps
        return out


class Block:
    """The attention block: attn_qkv_proj_fwd (RoPE, head split), attn_prefill_fwd (causal, rotation off),
    attn_out_proj_fwd, on the Llama-3-8B shape (inputs resident); each kernel timed."""

    def __init__(self, dev, bd, W, torch):
        self.pw, self.aw, self.bd = W.PROJ_LLAMA3_8B, W.LLAMA3_8B, bd
        pw = self.pw
        inp = W.proj_inputs(pw)
        self.x, self.wq, self.wo = inp.x.to(dev), inp.w_qkv.to(dev), inp.w_o.to(dev)
        bf = torch.bfloat16
        self.q = torch.empty(pw.B, pw.H, pw.T, pw.hd, dtype=bf, device=dev)
        self.k = torch.empty(pw.B, pw.KV, pw.T, pw.hd, dtype=bf, device=dev)
        self.v = torch.empty(pw.B, pw.KV, pw.T, pw.hd, dtype=bf, device=dev)
        self.o = torch.empty(pw.B, pw.H, pw.T, pw.hd, dtype=bf, device=dev)
        self.y = torch.empty(pw.B, pw.T, pw.D, dtype=bf, device=dev)

    def flops(self):
        return self.pw.qkv_flops() + self.aw.flops() + self.pw.out_flops()

    def __call__(self, stream, ev_qkv=None, ev_attn=None, ev_out=None):
        pw, bd = self.pw, self.bd
        if ev_qkv:
            bd.attn_set_timing_events(*ev_qkv)
        st = bd.attn_qkv_proj_fwd(self.x.data_ptr(), self.wq.data_ptr(), self.q.data_ptr(), self.k.data_ptr(),
                                  self.v.data_ptr(), pw.B, pw.T, pw.D, pw.H, pw.KV, pw.hd, 0, pw.rope_base,
                                  bd.ATTN_DTYPE_BF16, stream)
        if st != bd.ATTN_OK:
            raise RuntimeError(f"attn_qkv_proj_fwd: {bd.attn_status_str(st)} {bd.attn_last_error()}")
        if ev_attn:
            bd.attn_set_timing_events(*ev_attn)
        st = bd.attn_prefill_fwd(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.o.data_ptr(), None,
                                 pw.B, pw.T, pw.H, pw.KV, pw.hd, 0, 0.0, 1, 0, bd.ATTN_DTYPE_BF16,
                                 bd.ATTN_DTYPE_BF16, None, 0, stream)
        if st != bd.ATTN_OK:
            raise RuntimeError(f"attn_prefill_fwd: {bd.attn_status_str(st)} {bd.attn_last_error()}")
        if ev_out:
            bd.attn_set_timing_events(*ev_out)
        st = bd.attn_out_proj_fwd(self.o.data_ptr(), self.wo.data_ptr(), self.y.data_ptr(), pw.B, pw.T, pw.H, pw.hd,
                                  pw.D, bd.ATTN_DTYPE_BF16, bd.ATTN_DTYPE_BF16, stream)
        if st != bd.ATTN_OK:
            raise RuntimeError(f"attn_out_proj_fwd: {bd.attn_status_str(st)} {bd.attn_last_error()}")


class Backward:
    """attn_prefill_bwd on the forward's own out/lse (computed once, untimed)."""

    def __init__(self, w, dev, bd, W, torch, stream):
        self.w, self.bd = w, bd
        self.fwd = Prefill(w, dev, bd, W, torch)
        self.fwd(stream)
        self.dout = W.prefill_dout(w).to(dev)
        shp_q, shp_k = (w.B, w.H, w.T, w.hd), (w.B, w.KV, w.T, w.hd)
        self.dq = torch.empty(shp_q, dtype=torch.bfloat16, device=dev)
        self.dk = torch.empty(shp_k, dtype=torch.bfloat16, device=dev)
        self.dv = torch.empty(shp_k, dtype=torch.bfloat16, device=dev)
        self.ws_bytes = bd.attn_prefill_bwd_workspace_bytes(w.B, w.T, w.H, w.KV, w.hd, self.fwd.dt, w.rope_base)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev)

    def __call__(self, stream, events=None):
        w, bd, f = self.w, self.bd, self.fwd
        if events:
            bd.attn_set_timing_events(*events)
        st = bd.attn_prefill_bwd(f.q.data_ptr(), f.k.data_ptr(), f.v.data_ptr(), f.out.data_ptr(), f.lse.data_ptr(),
                                 self.dout.data_ptr(), self.dq.data_ptr(), self.dk.data_ptr(), self.dv.data_ptr(),
                                 w.B, w.T, w.H, w.KV, w.hd, w.pos0, w.rope_base, int(w.causal), w.alibi, f.dt,
                                 bd.ATTN_DTYPE_BF16, bd.ATTN_DTYPE_BF16, self.ws.data_ptr(), self.ws_bytes, stream)
        if st != bd.ATTN_OK:
            raise RuntimeError(f"attn_prefill_bwd: {bd.attn_status_str(st)} {bd.attn_last_error()}")

    def work(self):
        return self.w.bwd_flops()


def host_info():
    """Host CPU count and model (from /proc/cpuinfo) for the CPU-baseline records."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_cpus": os.cpu_count(), "cpu_model": model}


def measure_ceilings(torch, dev, mfma, hbm):
    """Same-run context for the rooflines, measured before the timed steps (the
    heavy work also brings the clock to its steady state first).

    mfma: the vendor GEMM (torch.matmul -> hipBLASLt) on N(0,1) bf16 operands.
    The published 2.5 PFLOP/s assumes the 2.4 GHz peak clock; with random data
    the chip runs power-limited well below it.
    hbm: a read-only stream of 4 GiB (libattn_probe.so: non-temporal 16-byte
    loads, every byte read once) and a torch copy of 2 GiB.
    """
    res = {}
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    if mfma:
        n = 8192
        g = torch.Generator(device=dev).manual_seed(11)
        a_ = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
        b_ = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
        for _ in range(10):
            c_ = a_ @ b_
        e0, e1 = ev(), ev()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            c_ = a_ @ b_
        e1.record()
        torch.cuda.synchronize()
        res["gemm_bf16_tflops"] = 2.0 * n ** 3 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12
        res["gemm"] = f"torch.matmul {n}x{n}x{n} bf16, N(0,1) operands"
        del a_, b_, c_
    if hbm:
        probe = ctypes.CDLL(os.path.join(ROOT, "transformer_attention_02_amd", "libattn_probe.so"))
        probe.attn_probe_read_stream.restype = ctypes.c_int
        probe.attn_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        probe.attn_probe_sink_words.restype = ctypes.c_size_t
        x_ = torch.ones(1 << 31, dtype=torch.bfloat16, device=dev)
        sink = torch.empty(probe.attn_probe_sink_words(), dtype=torch.int32, device=dev)
        nb = x_.numel() * x_.element_size()
        stream = torch.cuda.current_stream().cuda_stream
        run = lambda: probe.attn_probe_read_stream(x_.data_ptr(), nb, sink.data_ptr(), stream)  # noqa: E731
        for _ in range(5):
            assert run() == 0
        e0, e1 = ev(), ev()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            run()
        e1.record()
        torch.cuda.synchronize()
        res["hbm_read_stream_gbs"] = nb / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
        res["hbm_read_stream"] = ("read-only stream of 4 GiB, non-temporal 16-byte loads, 16384 x 512 threads, 8 loads in "
                                  "flight per thread (libattn_probe.so)")
        y_ = torch.empty(1 << 30, dtype=torch.bfloat16, device=dev)
        src = x_[: y_.numel()]
        for _ in range(3):
            y_.copy_(src)
        e0, e1 = ev(), ev()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            y_.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        res["hbm_copy_gbs"] = 2 * y_.numel() * 2 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
        res["hbm_copy"] = "torch copy of 2 GiB (read + write bytes)"
        del x_, y_, sink
    return res


def cpu_baseline_leg(pre, dec, heads, seqs):
    """The fp64 oracle on a bounded sample of the same workload (rank 0, N=1 only)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import attention_decode, attention_prefill

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    res = {"kind": "oracle", "cores": threads, **host_info()}
    f64 = lambda t: t.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
    if pre is not None:
        w = pre.w
        g = w.H // w.KV
        heads = max(g, heads // g * g)
        qs, ks, vs = f64(pre.q[0:1, :heads]), f64(pre.k[0:1, :heads // g]), f64(pre.v[0:1, :heads // g])
        t0 = time.perf_counter()
        ref, _ = attention_prefill(qs, ks, vs, pos0=w.pos0, rope_base=w.rope_base, causal=w.causal, alibi=w.alibi,
                                   q_offset=w.q_offset, window=w.window)
        dt = time.perf_counter() - t0
        flops = 4.0 * heads * w.hd * w.pairs()
        err = float(np.abs(f64(pre.out[0:1, :heads]) - ref).max())
        res.update(value=flops / dt / 1e12, unit="TFLOP/s", seconds=dt,
                   sample=f"{heads} query heads of batch 0 ({heads // g} KV heads), all {w.rows} query rows: "
                          f"{flops / w.flops() * 100:.2f}% of the prefill step",
                   max_abs_err_vs_gpu_bf16_out=err)
    if dec is not None:
        w = dec.w
        lens = dec.inp.lens
        pick = list(range(min(seqs, w.B)))
        t_total = 0.0
        nbytes = 0
        errs = []
        for b in pick:
            L = int(lens[b])
            kc = f64(dec.kc[b:b + 1, :, :L])
            vc = f64(dec.vc[b:b + 1, :, :L])
            t0 = time.perf_counter()
            ref, _, _, _ = attention_decode(f64(dec.q[b:b + 1]), f64(dec.kn[b:b + 1]), f64(dec.vn[b:b + 1]), kc, vc,
                                            np.array([L], dtype=np.int32), rope_base=w.rope_base, alibi=w.alibi)
            t_total += time.perf_counter() - t0
            nbytes += (L + 1) * w.KV * w.hd * 2 * 2
            errs.append(float(np.abs(f64(dec.out[b:b + 1]) - ref).max()))
        res["decode"] = {"value": nbytes / t_total / 1e9, "unit": "GB/s", "seconds": t_total,
                         "sample": f"sequences 0..{len(pick) - 1} of {w.B}", "max_abs_err_vs_gpu_bf16_out": max(errs)}
        if pre is None:
            res.update(value=res["decode"]["value"], unit="GB/s", seconds=t_total, sample=res["decode"]["sample"])
    return res


def cpu_baseline_fp8(dec8, seqs):
    """The fp64 oracle of the fp8-cache decode step, one sequence at a time."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention_decode_fp8

    w, inp = dec8.w, dec8.inp
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    f64 = lambda t: t.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
    pick = list(range(min(seqs, w.B)))
    t_total, nbytes, errs = 0.0, 0, []
    for b in pick:
        L = int(inp.lens[b])
        kc = dec8.kc[b:b + 1, :, :L].cpu().numpy()
        vc = dec8.vc[b:b + 1, :, :L].cpu().numpy()
        t0 = time.perf_counter()
        ref = attention_decode_fp8(f64(dec8.q[b:b + 1]), f64(dec8.kn[b:b + 1]), f64(dec8.vn[b:b + 1]), kc, vc,
                                   np.array([L], dtype=np.int32), w.k_scale, w.v_scale, rope_base=w.rope_base,
                                   alibi=w.alibi)[0]
        t_total += time.perf_counter() - t0
        nbytes += (L + 1) * w.KV * w.hd * 2
        errs.append(float(np.abs(f64(dec8.out[b:b + 1]) - ref).max()))
    return {"kind": "oracle", "cores": threads, **host_info(), "value": nbytes / t_total / 1e9,
            "unit": "GB/s", "seconds": t_total, "sample": f"sequences 0..{len(pick) - 1} of {w.B}",
            "max_abs_err_vs_gpu_bf16_out": max(errs)}


def cpu_baseline_latent(lat, seqs):
    """The fp64 oracle of the latent decode step (explicit per-head keys and values) on the first sequences."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention_decode_latent

    w, inp = lat.w, lat.inp
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    f64 = lambda t: t.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
    pick = list(range(min(seqs, w.B)))
    wk, wv = f64(lat.wk), f64(lat.wv)
    t_total, nbytes, errs = 0.0, 0, []
    for b in pick:
        L = int(inp.lens[b])
        cc = f64(lat.cc[b:b + 1, :L])
        t0 = time.perf_counter()
        ref = attention_decode_latent(f64(lat.q[b:b + 1]), f64(lat.cn[b:b + 1]), cc, np.array([L], dtype=np.int32),
                                      wk, wv, alibi=w.alibi)[0]
        t_total += time.perf_counter() - t0
        nbytes += (L + 1) * w.dc * 2
        errs.append(float(np.abs(f64(lat.out[b:b + 1]) - ref).max()))
    return {"kind": "oracle", "cores": threads, **host_info(), "value": nbytes / t_total / 1e9,
            "unit": "GB/s", "seconds": t_total, "sample": f"sequences 0..{len(pick) - 1} of {w.B}",
            "max_abs_err_vs_gpu_bf16_out": max(errs)}


def cpu_baseline_proj(pj, seqs):
    """The fp64 oracle of both projections (numpy matmul, RoPE, head split / merge) on the first sequences,
    checked against the GPU's outputs."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import out_projection, qkv_projection

    w = pj.w
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    f64 = lambda t: t.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
    wq, wo = f64(pj.wq), f64(pj.wo)
    n = min(seqs, w.B)
    secs, err = 0.0, 0.0
    for b in range(n):
        x, o = f64(pj.x[b:b + 1]), f64(pj.o[b:b + 1])
        t0 = time.perf_counter()
        q, k, v = qkv_projection(x, wq, H=w.H, KV=w.KV, hd=w.hd, rope_base=w.rope_base)
        y = out_projection(o, wo)
        secs += time.perf_counter() - t0
        err = max(err, float(np.abs(f64(pj.q[b:b + 1]) - q).max()), float(np.abs(f64(pj.k[b:b + 1]) - k).max()),
                  float(np.abs(f64(pj.v[b:b + 1]) - v).max()), float(np.abs(f64(pj.y[b:b + 1]) - y).max()))
    flops = n * w.T * (2.0 * w.N_qkv * w.D + 2.0 * w.D * w.H * w.hd)
    return {"kind": "oracle", "cores": threads, **host_info(), "value": flops / secs / 1e12,
            "unit": "TFLOP/s", "seconds": secs, "sample": f"sequences 0..{n - 1} of {w.B} (both projections)",
            "max_abs_err_vs_gpu_bf16": err}


def cpu_baseline_block(blk, tokens):
    """The fp64 oracle of the block (projection with RoPE, causal attention, output projection) on the first
    tokens of sequence 0; with a causal mask those output rows depend on those tokens only, so they are
    checked against the GPU's rows."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention_prefill, out_projection, qkv_projection

    pw = blk.pw
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    f64 = lambda t: t.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
    T = min(tokens, pw.T)
    x, wq, wo = f64(blk.x[:1, :T]), f64(blk.wq), f64(blk.wo)
    t0 = time.perf_counter()
    q, k, v = qkv_projection(x, wq, H=pw.H, KV=pw.KV, hd=pw.hd, rope_base=pw.rope_base)
    o, _ = attention_prefill(q, k, v, rope_base=0.0, causal=True)
    y = out_projection(o, wo)
    secs = time.perf_counter() - t0
    flops = 2.0 * T * pw.N_qkv * pw.D + 4.0 * pw.H * pw.hd * T * (T + 1) / 2 + 2.0 * T * pw.D * pw.H * pw.hd
    err = float(np.abs(f64(blk.y[:1, :T]) - y).max())
    return {"kind": "oracle", "cores": threads, **host_info(), "value": flops / secs / 1e12,
            "unit": "TFLOP/s", "seconds": secs, "sample": f"the block on tokens 0..{T - 1} of sequence 0",
            "max_abs_err_vs_gpu_bf16": err}


def cpu_baseline_bwd(bwd, heads):
    """The fp64 oracle backward on a bounded sample: the first ``heads`` query
    heads (whole GQA groups) of batch 0, all rows."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention_prefill_bwd

    w, f = bwd.w, bwd.fwd
    g = w.H // w.KV
    heads = max(g, heads // g * g)
    f64 = lambda t: t.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    qs, ks, vs = f64(f.q[0:1, :heads]), f64(f.k[0:1, :heads // g]), f64(f.v[0:1, :heads // g])
    t0 = time.perf_counter()
    dq, _, _ = attention_prefill_bwd(qs, ks, vs, f64(bwd.dout[0:1, :heads]), pos0=w.pos0, rope_base=w.rope_base,
                                     causal=w.causal, alibi=w.alibi)
    dt = time.perf_counter() - t0
    flops = 10.0 * heads * w.hd * w.pairs()
    err = float(np.abs(f64(bwd.dq[0:1, :heads]) - dq).max())
    return {"kind": "oracle", "cores": threads, **host_info(), "value": flops / dt / 1e12,
            "unit": "TFLOP/s", "seconds": dt,
            "sample": f"{heads} query heads of batch 0 ({heads // g} KV heads), all {w.T} rows: "
                      f"{flops / w.bwd_flops() * 100:.2f}% of the backward step",
            "max_abs_err_dq_vs_gpu_bf16": err}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all",
                    choices=["all", "prefill", "decode", "decode-fp8", "latent-decode", "proj", "block", "alibi",
                             "small", "window", "chunk", "backward", "copy"],
                    help="copy: a plain 1 GiB device copy, the reference for scaling HBM byte counters")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the same-run ceilings measured before the timed steps: the library GEMM (practical "
                         "bf16 matrix-core ceiling) and the read-only HBM stream")
    ap.add_argument("--cpu-heads", type=int, default=24)
    ap.add_argument("--cpu-seqs", type=int, default=64)
    ap.add_argument("--cpu-heads-bwd", type=int, default=16)
    ap.add_argument("--cpu-seqs-latent", type=int, default=8)
    ap.add_argument("--cpu-seqs-proj", type=int, default=4)
    ap.add_argument("--cpu-tokens-block", type=int, default=4096)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this path runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "sharding across GPUs is not implemented.", file=sys.stderr)
        sys.exit(2)

    import torch

    from transformer_attention_02_amd import binding as bd
    from transformer_attention_02_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    bd.load()
    dev = torch.device("cuda:0")
    hip = HipEvents()

    if args.workload == "copy":
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        nbytes = 2 * src.numel() * src.element_size()
        print(json.dumps({"workload": "copy", "bytes_read": nbytes // 2, "bytes_written": nbytes // 2,
                          "ms": ms, "GB/s": nbytes / ms / 1e6}), flush=True)
        return

    pre_w = {"all": W.LLAMA3_8B, "prefill": W.LLAMA3_8B, "alibi": W.ALIBI_MHA, "small": W.SMALL_BF16,
             "window": W.LLAMA3_WINDOW, "chunk": W.LLAMA3_CHUNK}.get(args.workload)
    pre = Prefill(pre_w, dev, bd, W, torch) if pre_w is not None else None
    dec = Decode(W.KV_DECODE, dev, bd, W, torch) if args.workload in ("all", "decode", "decode-fp8") else None
    dec8 = DecodeFp8(W.KV_DECODE_FP8, dev, bd, W, torch) if args.workload == "decode-fp8" else None
    lat = LatentDecode(W.LATENT_DECODE, dev, bd, W, torch) if args.workload == "latent-decode" else None
    pj = Proj(W.PROJ_LLAMA3_8B, dev, bd, W, torch) if args.workload == "proj" else None
    blk = Block(dev, bd, W, torch) if args.workload == "block" else None
    stream = torch.cuda.current_stream().cuda_stream
    bwd = Backward(W.LLAMA3_8B, dev, bd, W, torch, stream) if args.workload == "backward" else None
    log(f"inputs ready: prefill={pre_w.name if pre else None} decode={dec.w.name if dec else None} "
        f"backward={bwd.w.name if bwd else None}")
    ceilings = None
    if not args.no_ceilings and (pre or bwd or dec or dec8 or lat):
        ceilings = measure_ceilings(torch, dev, mfma=bool(pre or bwd), hbm=bool(dec or dec8 or lat))
        log(f"same-run ceilings: {ceilings}")

    for _ in range(args.warmup):
        if pre:
            pre(stream)
        if dec:
            dec(stream)
        if bwd:
            bwd(stream)
        if dec8:
            dec8(stream)
        if lat:
            lat(stream)
        if pj:
            pj(stream)
        if blk:
            blk(stream)
    torch.cuda.synchronize()

    K = args.steps
    ev = {k: [(hip.create(), hip.create()) for _ in range(K)] for k in ("pc", "pk", "dc", "dk", "bc", "bk", "ec", "ek", "lc", "lk",
                                                                     "jc", "jq", "jo", "xc", "xq", "xa", "xo")}
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(K):
        if pre:
            hip.hip.hipEventRecord(ctypes.c_void_p(ev["pc"][i][0]), ctypes.c_void_p(stream))
            pre(stream, ev["pk"][i])
            hip.hip.hipEventRecord(ctypes.c_void_p(ev["pc"][i][1]), ctypes.c_void_p(stream))
        if dec:
            hip.hip.hipEventRecord(ctypes.c_void_p(ev["dc"][i][0]), ctypes.c_void_p(stream))
            dec(stream, ev["dk"][i])
            hip.hip.hipEventRecord(ctypes.c_void_p(ev["dc"][i][1]), ctypes.c_void_p(stream))
        if lat:
            hip.hip.hipEventRecord(ctypes.c_void_p(ev["lc"][i][0]), ctypes.c_void_p(stream))
            lat(stream, ev["lk"][i])
            hip.hip.hipEventRecord(ctypes.c_void_p(ev["lc"][i][1]), ctypes.c_void_p(stream))
        if pj:
            hip.hip.hipEventRecord(ctypes.c_void_p(ev["jc"][i][0]), ctypes.c_void_p(stream))
            pj(stream, ev["jq"][i], ev["jo"][i])
            hip.hip.hipEventRecord(ctypes.c_void_p(ev["jc"][i][1]), ctypes.c_void_p(stream))
        if blk:
            hip.hip.hipEventRecord(ctypes.c_void_p(ev["xc"][i][0]), ctypes.c_void_p(stream))
            blk(stream, ev["xq"][i], ev["xa"][i], ev["xo"][i])
            hip.hip.hipEventRecord(ctypes.c_void_p(ev["xc"][i][1]), ctypes.c_void_p(stream))
        if dec8:
            hip.hip.hipEventRecord(ctypes.c_void_p(ev["ec"][i][0]), ctypes.c_void_p(stream))
            dec8(stream, ev["ek"][i])
            hip.hip.hipEventRecord(ctypes.c_void_p(ev["ec"][i][1]), ctypes.c_void_p(stream))
        if bwd:
            hip.hip.hipEventRecord(ctypes.c_void_p(ev["bc"][i][0]), ctypes.c_void_p(stream))
            bwd(stream, ev["bk"][i])
            hip.hip.hipEventRecord(ctypes.c_void_p(ev["bc"][i][1]), ctypes.c_void_p(stream))
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)

    def avg(key):
        return sum(hip.elapsed_ms(a, b) for a, b in ev[key]) / K

    def med_min(key):
        v = sorted(hip.elapsed_ms(a, b) for a, b in ev[key])
        return v[len(v) // 2], v[0]

    line = {"metric": METRIC, "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": total_ms / K,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) bf16; random lengths for decode)"}
    cfg = {}
    if pre:
        w = pre.w
        pc, pk = avg("pc"), avg("pk")
        tflops = w.flops() / (pc * 1e-3) / 1e12
        kt = w.flops() / (pk * 1e-3) / 1e12
        line.update(value=tflops, unit="TFLOP/s")
        cfg["workload"] = w.name
        cfg["prefill"] = {"B": w.B, "T": w.T, "H": w.H, "KV": w.KV, "hd": w.hd, "rope_base": w.rope_base,
                          "causal": w.causal, "alibi": w.alibi, "out_dtype": "bf16", "flops": w.flops(),
                          "call_ms": pc, "kernel_ms": pk}
        if w.Tq or w.q_offset or w.window:
            cfg["prefill"].update(query_rows=w.rows, q_offset=w.q_offset, window=w.window)
        cfg["prefill"]["kernel_ms_median"], cfg["prefill"]["kernel_ms_min"] = med_min("pk")
        traffic = traffic_for("prefill_mfma_kernel", PREFILL_SOURCES, w.name)
        # frac is the attention kernel's; frac_call counts the whole call, the K
        # rotation pre-pass included
        line["roofline"] = {"bound": "mfma", "achieved": kt, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                            "frac": kt / PEAK_BF16_TFLOPS, "traffic": traffic,
                            "kernel": f"prefill_mfma_kernel<{w.hd}>", "frac_call": tflops / PEAK_BF16_TFLOPS}
    if dec:
        w = dec.w
        dc, dk = avg("dc"), avg("dk")
        gbs = w.kv_read_bytes() / (dc * 1e-3) / 1e9
        kg = w.kv_read_bytes() / (dk * 1e-3) / 1e9
        dline = {"value": gbs, "unit": "GB/s", "call_ms": dc, "kernel_ms": dk, "kv_bytes": w.kv_read_bytes(),
                 "roofline": {"bound": "hbm", "achieved": kg, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": kg / PEAK_HBM_GBS, "traffic": traffic_for("decode_split", DECODE_SOURCES, w.name),
                              "kernel": f"decode_split_mfma_kernel<{w.hd}>"}}
        dline["kernel_ms_median"], dline["kernel_ms_min"] = med_min("dk")
        cfg["decode"] = {"B": w.B, "H": w.H, "KV": w.KV, "hd": w.hd, "len_range": [w.len_lo, w.len_hi],
                         "len_seed": w.len_seed, "Lmax": dec.Lmax, "rope_base": w.rope_base, "out_dtype": "bf16"}
        line["decode"] = dline
        if not pre:
            line.update(value=gbs, unit="GB/s", roofline=dline["roofline"])
            cfg["workload"] = w.name
        else:
            cfg["workload"] = cfg["workload"] + " + " + w.name
    if dec8:
        w = dec8.w
        ec, ek = avg("ec"), avg("ek")
        gbs = w.kv_read_bytes() / (ec * 1e-3) / 1e9
        kg = w.kv_read_bytes() / (ek * 1e-3) / 1e9
        bf = line.pop("decode")
        line.update(value=gbs, unit="GB/s", metric="fp8 E4M3 KV-cache decode: KV-read GB/s, 1 GPU")
        line["roofline"] = {"bound": "hbm", "achieved": kg, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": kg / PEAK_HBM_GBS,
                            "traffic": traffic_for("decode_split_fp8", DECODE_SOURCES, w.name),
                            "kernel": f"decode_split_mfma_kernel<{w.hd}, fp8>"}
        cfg["workload"] = w.name
        cfg["decode_fp8"] = {"B": w.B, "H": w.H, "KV": w.KV, "hd": w.hd, "k_scale": w.k_scale, "v_scale": w.v_scale,
                             "kv_bytes": w.kv_read_bytes(), "call_ms": ec, "kernel_ms": ek,
                             "tokens_per_s": w.B / (ec * 1e-3)}
        cfg["decode_fp8"]["kernel_ms_median"], cfg["decode_fp8"]["kernel_ms_min"] = med_min("ek")
        # before / after: the bf16-cache step of the same shape in the same run
        cfg["bf16_cache"] = {"call_ms": bf["call_ms"], "kernel_ms": bf["kernel_ms"], "GB/s": bf["value"],
                             "kv_bytes": bf["kv_bytes"], "tokens_per_s": W.KV_DECODE.B / (bf["call_ms"] * 1e-3)}
        line["speedup_vs_bf16_cache"] = bf["call_ms"] / ec
    if lat:
        w = lat.w
        lc, lk = avg("lc"), avg("lk")
        gbs = w.cache_read_bytes() / (lc * 1e-3) / 1e9
        kg = w.cache_read_bytes() / (lk * 1e-3) / 1e9
        line.update(value=gbs, unit="GB/s", metric="latent-cache decode: cache-read GB/s, 1 GPU")
        line["roofline"] = {"bound": "hbm", "achieved": kg, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": kg / PEAK_HBM_GBS, "traffic": traffic_for("latent_split", LATENT_SOURCES, w.name),
                            "kernel": f"latent_split_kernel<{w.dc}>"}
        cfg["workload"] = w.name
        cfg["latent_decode"] = {"B": w.B, "H": w.H, "hd": w.hd, "dc": w.dc, "len_range": [w.len_lo, w.len_hi],
                                "len_seed": w.len_seed, "Lmax": lat.Lmax, "cache_bytes": w.cache_read_bytes(),
                                "weight_bytes": 2 * w.H * w.dc * w.hd * 2, "call_ms": lc, "kernel_ms": lk,
                                "tokens_per_s": w.B / (lc * 1e-3)}
        cfg["latent_decode"]["kernel_ms_median"], cfg["latent_decode"]["kernel_ms_min"] = med_min("lk")
    if pj:
        w = pj.w
        jc, jq, jo = avg("jc"), avg("jq"), avg("jo")
        fl = w.qkv_flops() + w.out_flops()
        kq = w.qkv_flops() / (jq * 1e-3) / 1e12
        line.update(value=fl / (jc * 1e-3) / 1e12, unit="TFLOP/s",
                    metric="QKV projection (RoPE, head split) + output projection TFLOP/s, 1 GPU")
        cfg["workload"] = w.name
        lib = pj.library_gemms(torch)
        cfg["proj"] = {"B": w.B, "T": w.T, "D": w.D, "H": w.H, "KV": w.KV, "hd": w.hd, "rope_base": w.rope_base,
                       "qkv_flops": w.qkv_flops(), "out_flops": w.out_flops(), "call_ms": jc,
                       "qkv_kernel_ms": jq, "out_kernel_ms": jo,
                       "qkv_kernel_tflops": kq, "out_kernel_tflops": w.out_flops() / (jo * 1e-3) / 1e12,
                       "library_gemm_ms": lib,
                       "library_gemm": "torch.matmul of the same operands (x w_qkv^T, o' w_o^T): plain GEMMs, "
                                       "no rotation or head split"}
        cfg["proj"]["qkv_kernel_ms_median"], cfg["proj"]["qkv_kernel_ms_min"] = med_min("jq")
        line["roofline"] = {"bound": "mfma", "achieved": kq, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                            "frac": kq / PEAK_BF16_TFLOPS, "traffic": traffic_for("proj_qkv", PROJ_SOURCES, w.name),
                            "kernel": "proj_gemm_kernel<PROJ_QKV>"}
    if blk:
        pw, aw = blk.pw, blk.aw
        xc, xq, xa, xo = avg("xc"), avg("xq"), avg("xa"), avg("xo")
        line.update(value=blk.flops() / (xc * 1e-3) / 1e12, unit="TFLOP/s",
                    metric="attention block (QKV projection + RoPE, causal GQA attention, output projection) "
                           "TFLOP/s, 1 GPU")
        cfg["workload"] = "llama3-8b attention block B=4 T=4096 D=4096 H=32 KV=8 hd=128 rope=5e5"
        parts = {"qkv": (xq, pw.qkv_flops(), "proj_gemm_kernel<PROJ_QKV>"),
                 "attention": (xa, aw.flops(), "prefill_mfma_kernel<128>"),
                 "out": (xo, pw.out_flops(), "proj_gemm_kernel<PROJ_OUT>")}
        cfg["block"] = {"B": pw.B, "T": pw.T, "D": pw.D, "H": pw.H, "KV": pw.KV, "hd": pw.hd,
                        "rope_base": pw.rope_base, "flops": blk.flops(), "call_ms": xc,
                        "tokens_per_s": pw.B * pw.T / (xc * 1e-3),
                        "kernels": {k: {"ms": v[0], "tflops": v[1] / (v[0] * 1e-3) / 1e12} for k, v in parts.items()}}
        name = max(parts, key=lambda k: parts[k][0])
        ms, fl, kern = parts[name]
        kt = fl / (ms * 1e-3) / 1e12
        traffic = traffic_for("proj_qkv", PROJ_SOURCES, pw.name) if name == "qkv" else (
            traffic_for("proj_out", PROJ_SOURCES, pw.name) if name == "out" else None)
        line["roofline"] = {"bound": "mfma", "achieved": kt, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                            "frac": kt / PEAK_BF16_TFLOPS, "traffic": traffic, "kernel": kern}
    if bwd:
        w = bwd.w
        bc, bk = avg("bc"), avg("bk")
        tflops = w.bwd_flops() / (bc * 1e-3) / 1e12
        kt = w.bwd_flops() / (bk * 1e-3) / 1e12
        line.update(value=tflops, unit="TFLOP/s", metric="causal GQA+RoPE attn bwd TFLOP/s (prefill), 1 GPU")
        cfg["workload"] = "backward of " + w.name
        cfg["backward"] = {"B": w.B, "T": w.T, "H": w.H, "KV": w.KV, "hd": w.hd, "rope_base": w.rope_base,
                           "causal": w.causal, "grad_dtype": "bf16", "flops": w.bwd_flops(), "call_ms": bc,
                           "kernels_ms": bk}
        cfg["backward"]["kernels_ms_median"], cfg["backward"]["kernels_ms_min"] = med_min("bk")
        line["roofline"] = {"bound": "mfma", "achieved": kt, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                            "frac": kt / PEAK_BF16_TFLOPS,
                            "traffic": traffic_for("backward_mfma", BACKWARD_SOURCES, cfg["workload"]),
                            "kernel": f"bwd_dq_mfma_kernel<{w.hd}> + bwd_dkv_mfma_kernel<{w.hd}> (timed together)"}
    line["config"] = cfg
    torch.cuda.synchronize()
    ok = True
    if pre:
        ok &= bool(torch.isfinite(pre.out).all().item())
    if dec:
        ok &= bool(torch.isfinite(dec.out).all().item())
    if dec8:
        ok &= bool(torch.isfinite(dec8.out).all().item())
    if lat:
        ok &= bool(torch.isfinite(lat.out).all().item())
    if pj:
        for t in (pj.q, pj.k, pj.v, pj.y):
            ok &= bool(torch.isfinite(t).all().item())
    if blk:
        ok &= bool(torch.isfinite(blk.y).all().item())
    if bwd:
        for t in (bwd.dq, bwd.dk, bwd.dv):
            ok &= bool(torch.isfinite(t).all().item())
    line["outputs_finite"] = ok
    hip.close()

    if ceilings is not None:
        mc = dict(ceilings)
        if (pre or bwd) and "gemm_bf16_tflops" in mc:
            mc["prefill_kernel_vs_gemm" if pre else "kernel_vs_gemm"] = line["roofline"]["achieved"] / mc["gemm_bf16_tflops"]
        dk = line.get("decode", {}).get("roofline", {}).get("achieved") if pre else (
            line["roofline"]["achieved"] if (dec or dec8 or lat) else None)
        if dk and "hbm_read_stream_gbs" in mc:
            mc["decode_kernel_vs_read_stream"] = dk / mc["hbm_read_stream_gbs"]
        line["measured_ceilings"] = mc

    if not args.no_cpu_baseline and blk:
        log("cpu baseline: timing the fp64 oracle block on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline_block(blk, args.cpu_tokens_block)
    elif not args.no_cpu_baseline and pj:
        log("cpu baseline: timing the fp64 oracle projections on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline_proj(pj, args.cpu_seqs_proj)
    elif not args.no_cpu_baseline and lat:
        log("cpu baseline: timing the fp64 oracle latent decode on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline_latent(lat, args.cpu_seqs_latent)
    elif not args.no_cpu_baseline and dec8:
        log("cpu baseline: timing the fp64 oracle fp8 decode on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline_fp8(dec8, args.cpu_seqs)
    elif not args.no_cpu_baseline and bwd:
        log("cpu baseline: timing the fp64 oracle backward on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline_bwd(bwd, args.cpu_heads_bwd)
    elif not args.no_cpu_baseline:
        log("cpu baseline: timing the fp64 oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline_leg(pre, dec, args.cpu_heads, args.cpu_seqs)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
