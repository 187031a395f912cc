"""ctypes binding of libattn.so (argument marshalling only).

The raw functions keep the C names and signatures of ``include/attn.h``
(pointers are Python ints). :func:`prefill` and :func:`decode` accept torch
tensors already on the GPU, allocate the outputs and workspace with torch (the
memory and streams are torch's; every step of the computation runs in the
library's HIP kernels) and raise :class:`AttnError` on a non-OK status.

There is no fallback: if the library is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# ATTN_LIB selects another build of the same library (the sanitizer build of
# the checks); there is no fallback either way.
LIB_PATH = os.environ.get("ATTN_LIB") or os.path.join(PKG, "libattn.so")

ATTN_OK = 0
ATTN_ERR_NULL = 1
ATTN_ERR_SHAPE = 2
ATTN_ERR_UNSUPPORTED = 3
ATTN_ERR_ALIGN = 4
ATTN_ERR_WORKSPACE = 5
ATTN_ERR_HIP = 6

ATTN_DTYPE_F32 = 0
ATTN_DTYPE_BF16 = 1

ATTN_ALIBI_NONE = 0
ATTN_ALIBI_GEOMETRIC = 1
ATTN_ALIBI_PAGE1 = 2

EXPORTS = (
    "attn_abi_version",
    "attn_status_str",
    "attn_last_error",
    "attn_set_timing_events",
    "attn_prefill_workspace_bytes",
    "attn_prefill_fwd",
    "attn_prefill_ex_fwd",
    "attn_prefill_bwd_workspace_bytes",
    "attn_prefill_bwd",
    "attn_decode_workspace_bytes",
    "attn_decode_fwd",
    "attn_decode_fwd_noalloc",
    "attn_decode_fp8_fwd",
    "attn_decode_latent_workspace_bytes",
    "attn_decode_latent_fwd",
    "attn_qkv_proj_fwd",
    "attn_qkv_proj_cache_fwd",
    "attn_out_proj_fwd",
)

_P = ctypes.c_void_p
_I = ctypes.c_int
_D = ctypes.c_double
_S = ctypes.c_size_t
_F = ctypes.c_float

_SIGS = {
    "attn_abi_version": (_I, []),
    "attn_status_str": (ctypes.c_char_p, [_I]),
    "attn_last_error": (ctypes.c_char_p, []),
    "attn_set_timing_events": (_I, [_P, _P]),
    "attn_prefill_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _D]),
    "attn_prefill_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _D, _I, _I, _I, _I, _P, _S, _P]),
    "attn_prefill_ex_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _D, _I, _I, _I, _I, _P, _S,
                                 _P]),
    "attn_prefill_bwd_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I, _D]),
    "attn_prefill_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _D, _I, _I, _I, _I, _I, _P,
                              _S, _P]),
    "attn_decode_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "attn_decode_fwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _D, _I, _I, _I, _P, _S, _P]),
    "attn_decode_fwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _D, _I, _I, _I, _P]),
    "attn_decode_fp8_fwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _D, _I, _F, _F, _I, _I, _P, _S,
                                 _P]),
    "attn_decode_latent_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "attn_decode_latent_fwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _S, _P]),
    "attn_qkv_proj_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _D, _I, _P]),
    "attn_qkv_proj_cache_fwd": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _D, _I, _P]),
    "attn_out_proj_fwd": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_str(status)}: {detail}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Open libattn.so (once) and declare its signatures. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is not built; run `python -m transformer_attention_02_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def attn_abi_version() -> int:
    return load().attn_abi_version()


def attn_status_str(status: int) -> str:
    return load().attn_status_str(status).decode()


status_str = attn_status_str


def attn_last_error() -> str:
    return load().attn_last_error().decode()


def attn_set_timing_events(start, stop) -> int:
    return load().attn_set_timing_events(start, stop)


def attn_prefill_workspace_bytes(B, T, KV, hd, dtype, rope_base) -> int:
    return load().attn_prefill_workspace_bytes(B, T, KV, hd, dtype, float(rope_base))


def attn_prefill_fwd(q, k, v, out, lse, B, T, H, KV, hd, pos0, rope_base, causal, alibi, dtype, out_dtype,
                     workspace, workspace_bytes, stream) -> int:
    return load().attn_prefill_fwd(q, k, v, out, lse, B, T, H, KV, hd, pos0, float(rope_base), causal, alibi,
                                   dtype, out_dtype, workspace, workspace_bytes, stream)


def attn_prefill_ex_fwd(q, k, v, out, lse, B, Tq, Tk, H, KV, hd, pos0, q_offset, window, rope_base, causal, alibi,
                        dtype, out_dtype, workspace, workspace_bytes, stream) -> int:
    return load().attn_prefill_ex_fwd(q, k, v, out, lse, B, Tq, Tk, H, KV, hd, pos0, q_offset, window,
                                      float(rope_base), causal, alibi, dtype, out_dtype, workspace, workspace_bytes,
                                      stream)


def attn_prefill_bwd_workspace_bytes(B, T, H, KV, hd, dtype, rope_base) -> int:
    return load().attn_prefill_bwd_workspace_bytes(B, T, H, KV, hd, dtype, float(rope_base))


def attn_prefill_bwd(q, k, v, out, lse, dout, dq, dk, dv, B, T, H, KV, hd, pos0, rope_base, causal, alibi, dtype,
                     out_dtype, grad_dtype, workspace, workspace_bytes, stream) -> int:
    return load().attn_prefill_bwd(q, k, v, out, lse, dout, dq, dk, dv, B, T, H, KV, hd, pos0, float(rope_base),
                                   causal, alibi, dtype, out_dtype, grad_dtype, workspace, workspace_bytes, stream)


def attn_decode_workspace_bytes(B, H, KV, hd, Lmax) -> int:
    return load().attn_decode_workspace_bytes(B, H, KV, hd, Lmax)


def attn_decode_fwd(q, k_new, v_new, k_cache, v_cache, cache_lens, out, lse, B, H, KV, hd, Lmax, rope_base, alibi,
                    dtype, out_dtype, workspace, workspace_bytes, stream) -> int:
    return load().attn_decode_fwd(q, k_new, v_new, k_cache, v_cache, cache_lens, out, lse, B, H, KV, hd, Lmax,
                                  float(rope_base), alibi, dtype, out_dtype, workspace, workspace_bytes, stream)


def attn_decode_fwd_noalloc(q, k_new, v_new, k_cache, v_cache, cache_lens, out, lse, B, H, KV, hd, Lmax, rope_base,
                            alibi, dtype, out_dtype, stream) -> int:
    return load().attn_decode_fwd_noalloc(q, k_new, v_new, k_cache, v_cache, cache_lens, out, lse, B, H, KV, hd, Lmax,
                                          float(rope_base), alibi, dtype, out_dtype, stream)


def attn_decode_fp8_fwd(q, k_new, v_new, k_cache, v_cache, cache_lens, out, lse, B, H, KV, hd, Lmax, rope_base, alibi,
                        k_scale, v_scale, dtype, out_dtype, workspace, workspace_bytes, stream) -> int:
    return load().attn_decode_fp8_fwd(q, k_new, v_new, k_cache, v_cache, cache_lens, out, lse, B, H, KV, hd, Lmax,
                                      float(rope_base), alibi, float(k_scale), float(v_scale), dtype, out_dtype,
                                      workspace, workspace_bytes, stream)


def attn_decode_latent_workspace_bytes(B, H, dc, Lmax) -> int:
    return load().attn_decode_latent_workspace_bytes(B, H, dc, Lmax)


def attn_decode_latent_fwd(q, c_new, c_cache, cache_lens, w_uk, w_uv, out, lse, B, H, hd, dc, Lmax, alibi, dtype,
                           out_dtype, workspace, workspace_bytes, stream) -> int:
    return load().attn_decode_latent_fwd(q, c_new, c_cache, cache_lens, w_uk, w_uv, out, lse, B, H, hd, dc, Lmax,
                                         alibi, dtype, out_dtype, workspace, workspace_bytes, stream)


def attn_qkv_proj_fwd(x, w_qkv, q, k, v, B, T, D, H, KV, hd, pos0, rope_base, dtype, stream) -> int:
    return load().attn_qkv_proj_fwd(x, w_qkv, q, k, v, B, T, D, H, KV, hd, pos0, float(rope_base), dtype, stream)


def attn_qkv_proj_cache_fwd(x, w_qkv, q, k_cache, v_cache, cache_lens, B, T, D, H, KV, hd, Lmax, rope_base, dtype,
                            stream) -> int:
    return load().attn_qkv_proj_cache_fwd(x, w_qkv, q, k_cache, v_cache, cache_lens, B, T, D, H, KV, hd, Lmax,
                                          float(rope_base), dtype, stream)


def attn_out_proj_fwd(o, w_o, y, B, T, H, hd, D, dtype, out_dtype, stream) -> int:
    return load().attn_out_proj_fwd(o, w_o, y, B, T, H, hd, D, dtype, out_dtype, stream)


# --------------------------------------------------------------- torch helpers
def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    if t.dtype == torch.float32:
        return ATTN_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(status: int):
    if status != ATTN_OK:
        raise AttnError(status, attn_last_error())


def _require(tensors: dict, dtype=None, same_dtype=True):
    """Check torch tensors before their raw pointers cross the C ABI.

    The library sees only pointers and sizes, so a strided view or a tensor of
    another dtype would be read with the wrong layout. ``tensors`` maps names
    to tensors (None entries are skipped); every tensor must be contiguous, of
    ``dtype`` when given, and (``same_dtype``) all of one dtype. Raises
    ValueError / TypeError before any launch; :func:`_require_gpu` then checks
    the device.
    """
    items = [(n, t) for n, t in tensors.items() if t is not None]
    for n, t in items:
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous (got strides {tuple(t.stride())} for shape {tuple(t.shape)})")
    for n, t in items:
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{n} must be {dtype} (got {t.dtype})")
    if same_dtype and items:
        d0 = items[0][1].dtype
        for n, t in items[1:]:
            if t.dtype != d0:
                raise TypeError(f"{n} is {t.dtype} but {items[0][0]} is {d0}")


def _require_gpu(*tensors):
    """Every tensor (None skipped) must live on the GPU: checked last, after layout, dtype and shape."""
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError(f"a {tuple(t.shape)} {t.dtype} operand must be a GPU tensor (got device {t.device})")


def _require_shape(name, t, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _stream_ptr(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def prefill_workspace(B, T, KV, hd, dtype_code, rope_base, device):
    import torch

    n = attn_prefill_workspace_bytes(B, T, KV, hd, dtype_code, rope_base)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device), n


def prefill(q, k, v, *, pos0=0, rope_base=10000.0, causal=True, alibi=ATTN_ALIBI_NONE, out_dtype=None,
            want_lse=True, out=None, lse=None, workspace=None, stream=None, q_offset=0, window=0):
    """Run the prefill forward on torch tensors q [B,H,Tq,hd], k/v [B,KV,Tk,hd] (same dtype, contiguous, on GPU).

    With Tq == Tk, q_offset == 0 and window == 0 this is attn_prefill_fwd; otherwise
    attn_prefill_ex_fwd (query chunk at token q_offset, sliding window). Returns
    (out, lse). ``out_dtype`` defaults to fp32.
    """
    import torch

    _require({"q": q, "k": k, "v": v})
    B, H, Tq, hd = q.shape
    KV, Tk = k.shape[1], k.shape[2]
    _require_shape("k", k, (B, KV, Tk, hd))
    _require_shape("v", v, (B, KV, Tk, hd))
    dt = _dtype_code(q)
    odt = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(B, H, Tq, hd, dtype=odt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(B, H, Tq, dtype=torch.float32, device=q.device)
    _require({"out": out})
    _require({"lse": lse}, dtype=torch.float32)
    _require_shape("out", out, (B, H, Tq, hd))
    _require_shape("lse", lse, (B, H, Tq))
    if workspace is None:
        workspace, nbytes = prefill_workspace(B, Tk, KV, hd, dt, rope_base, q.device)
    else:
        _require({"workspace": workspace})
        nbytes = workspace.numel() * workspace.element_size()
    _require_gpu(q, k, v, out, lse, workspace)
    lse_ptr = lse.data_ptr() if lse is not None else None
    if Tq == Tk and q_offset == 0 and window == 0:
        st = attn_prefill_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr, B, Tq, H, KV, hd,
                              pos0, rope_base, int(causal), alibi, dt, _dtype_code(out), workspace.data_ptr(), nbytes,
                              _stream_ptr(stream))
    else:
        st = attn_prefill_ex_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr, B, Tq, Tk, H, KV,
                                 hd, pos0, q_offset, window, rope_base, int(causal), alibi, dt, _dtype_code(out),
                                 workspace.data_ptr(), nbytes, _stream_ptr(stream))
    _check(st)
    return out, lse


def prefill_bwd(q, k, v, out, lse, dout, *, pos0=0, rope_base=10000.0, causal=True, alibi=ATTN_ALIBI_NONE,
                grad_dtype=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Run attn_prefill_bwd on GPU torch tensors: q [B,H,T,hd], k/v [B,KV,T,hd], the forward's out and
    lse, and dout (same dtype as out). Returns (dq, dk, dv); ``grad_dtype`` defaults to fp32."""
    import torch

    _require({"q": q, "k": k, "v": v})
    _require({"out": out, "dout": dout})
    _require({"lse": lse}, dtype=torch.float32)
    B, H, T, hd = q.shape
    KV = k.shape[1]
    for n_, t_, shp in (("k", k, (B, KV, T, hd)), ("v", v, (B, KV, T, hd)), ("out", out, (B, H, T, hd)),
                        ("dout", dout, (B, H, T, hd)), ("lse", lse, (B, H, T))):
        _require_shape(n_, t_, shp)
    dt = _dtype_code(q)
    gdt = torch.float32 if grad_dtype is None else grad_dtype
    if dq is None:
        dq = torch.empty(B, H, T, hd, dtype=gdt, device=q.device)
    if dk is None:
        dk = torch.empty(B, KV, T, hd, dtype=gdt, device=q.device)
    if dv is None:
        dv = torch.empty(B, KV, T, hd, dtype=gdt, device=q.device)
    _require({"dq": dq, "dk": dk, "dv": dv})
    for n_, t_, shp in (("dq", dq, (B, H, T, hd)), ("dk", dk, (B, KV, T, hd)), ("dv", dv, (B, KV, T, hd))):
        _require_shape(n_, t_, shp)
    if workspace is None:
        n = attn_prefill_bwd_workspace_bytes(B, T, H, KV, hd, dt, rope_base)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _require({"workspace": workspace})
    nbytes = workspace.numel() * workspace.element_size()
    _require_gpu(q, k, v, out, lse, dout, dq, dk, dv, workspace)
    st = attn_prefill_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, T, H, KV, hd, pos0, rope_base, int(causal),
                          alibi, dt, _dtype_code(out), _dtype_code(dq), workspace.data_ptr(), nbytes,
                          _stream_ptr(stream))
    _check(st)
    return dq, dk, dv


def decode_workspace(B, H, KV, hd, Lmax, device):
    import torch

    n = attn_decode_workspace_bytes(B, H, KV, hd, Lmax)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device), n


def _decode_shapes(B, H, KV, hd, Lmax, k_new, v_new, k_cache, v_cache, cache_lens):
    _require_shape("k_new", k_new, (B, KV, hd))
    _require_shape("v_new", v_new, (B, KV, hd))
    _require_shape("k_cache", k_cache, (B, KV, Lmax, hd))
    _require_shape("v_cache", v_cache, (B, KV, Lmax, hd))
    _require_shape("cache_lens", cache_lens, (B,))


def _decode_outputs(out, lse, B, H, hd):
    import torch

    _require({"out": out})
    _require({"lse": lse}, dtype=torch.float32)
    _require_shape("out", out, (B, H, hd))
    _require_shape("lse", lse, (B, H))


def decode(q, k_new, v_new, k_cache, v_cache, cache_lens, *, rope_base=10000.0, alibi=ATTN_ALIBI_NONE,
           out_dtype=None, want_lse=True, out=None, lse=None, workspace=None, stream=None):
    """Run attn_decode_fwd on GPU torch tensors (see include/attn.h for shapes). Returns (out, lse).

    k_new = v_new = None: slot cache_lens[b] already holds the new token (see attn_qkv_proj_cache_fwd)."""
    import torch

    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must both be given or both be None")
    _require({"q": q, "k_new": k_new, "v_new": v_new, "k_cache": k_cache, "v_cache": v_cache})
    _require({"cache_lens": cache_lens}, dtype=torch.int32)
    B, H, hd = q.shape
    KV, Lmax = k_cache.shape[1], k_cache.shape[2]
    _decode_shapes(B, H, KV, hd, Lmax, k_new, v_new, k_cache, v_cache, cache_lens)
    dt = _dtype_code(q)
    odt = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(B, H, hd, dtype=odt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(B, H, dtype=torch.float32, device=q.device)
    _decode_outputs(out, lse, B, H, hd)
    if workspace is None:
        workspace, nbytes = decode_workspace(B, H, KV, hd, Lmax, q.device)
    else:
        _require({"workspace": workspace})
        nbytes = workspace.numel() * workspace.element_size()
    _require_gpu(q, k_new, v_new, k_cache, v_cache, cache_lens, out, lse, workspace)
    st = attn_decode_fwd(q.data_ptr(), None if k_new is None else k_new.data_ptr(),
                         None if v_new is None else v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                         cache_lens.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None,
                         B, H, KV, hd, Lmax, rope_base, alibi, dt, _dtype_code(out), workspace.data_ptr(), nbytes,
                         _stream_ptr(stream))
    _check(st)
    return out, lse


def decode_fp8(q, k_new, v_new, k_cache, v_cache, cache_lens, k_scale, v_scale, *, rope_base=10000.0,
               alibi=ATTN_ALIBI_NONE, out_dtype=None, want_lse=True, out=None, lse=None, workspace=None, stream=None):
    """Run attn_decode_fp8_fwd: caches are uint8 tensors of E4M3 codes. Returns (out, lse)."""
    import torch

    _require({"q": q, "k_new": k_new, "v_new": v_new})
    _require({"k_cache": k_cache, "v_cache": v_cache}, dtype=torch.uint8)
    _require({"cache_lens": cache_lens}, dtype=torch.int32)
    B, H, hd = q.shape
    KV, Lmax = k_cache.shape[1], k_cache.shape[2]
    _decode_shapes(B, H, KV, hd, Lmax, k_new, v_new, k_cache, v_cache, cache_lens)
    odt = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(B, H, hd, dtype=odt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(B, H, dtype=torch.float32, device=q.device)
    _decode_outputs(out, lse, B, H, hd)
    if workspace is None:
        workspace, nbytes = decode_workspace(B, H, KV, hd, Lmax, q.device)
    else:
        _require({"workspace": workspace})
        nbytes = workspace.numel() * workspace.element_size()
    _require_gpu(q, k_new, v_new, k_cache, v_cache, cache_lens, out, lse, workspace)
    st = attn_decode_fp8_fwd(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
                             v_cache.data_ptr(), cache_lens.data_ptr(), out.data_ptr(),
                             lse.data_ptr() if lse is not None else None, B, H, KV, hd, Lmax, rope_base, alibi,
                             k_scale, v_scale, _dtype_code(q), _dtype_code(out), workspace.data_ptr(), nbytes,
                             _stream_ptr(stream))
    _check(st)
    return out, lse


def decode_latent(q, c_new, c_cache, cache_lens, w_uk, w_uv, *, alibi=ATTN_ALIBI_NONE, out_dtype=None,
                  want_lse=True, out=None, lse=None, workspace=None, stream=None):
    """Run attn_decode_latent_fwd on GPU torch tensors (bf16). Returns (out, lse)."""
    import torch

    _require({"q": q, "c_new": c_new, "c_cache": c_cache, "w_uk": w_uk, "w_uv": w_uv})
    _require({"cache_lens": cache_lens}, dtype=torch.int32)
    B, H, hd = q.shape
    Lmax, dc = c_cache.shape[1], c_cache.shape[2]
    for n_, t_, shp in (("c_new", c_new, (B, dc)), ("c_cache", c_cache, (B, Lmax, dc)), ("w_uk", w_uk, (H, dc, hd)),
                        ("w_uv", w_uv, (H, dc, hd)), ("cache_lens", cache_lens, (B,))):
        _require_shape(n_, t_, shp)
    odt = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(B, H, hd, dtype=odt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(B, H, dtype=torch.float32, device=q.device)
    _decode_outputs(out, lse, B, H, hd)
    if workspace is None:
        n = attn_decode_latent_workspace_bytes(B, H, dc, Lmax)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _require({"workspace": workspace})
    nbytes = workspace.numel() * workspace.element_size()
    _require_gpu(q, c_new, c_cache, cache_lens, w_uk, w_uv, out, lse, workspace)
    st = attn_decode_latent_fwd(q.data_ptr(), c_new.data_ptr(), c_cache.data_ptr(), cache_lens.data_ptr(),
                                w_uk.data_ptr(), w_uv.data_ptr(), out.data_ptr(),
                                lse.data_ptr() if lse is not None else None, B, H, hd, dc, Lmax, alibi,
                                _dtype_code(q), _dtype_code(out), workspace.data_ptr(), nbytes, _stream_ptr(stream))
    _check(st)
    return out, lse


def qkv_proj(x, w_qkv, H, KV, *, pos0=0, rope_base=10000.0, stream=None):
    """attn_qkv_proj_fwd on GPU bf16 tensors x [B,T,D], w_qkv [(H+2KV)hd, D]. Returns (q, k, v)."""
    import torch

    _require({"x": x, "w_qkv": w_qkv})
    B, T, D = x.shape
    hd = w_qkv.shape[0] // (H + 2 * KV)
    _require_shape("w_qkv", w_qkv, ((H + 2 * KV) * hd, D))
    _require_gpu(x, w_qkv)
    q = torch.empty(B, H, T, hd, dtype=torch.bfloat16, device=x.device)
    k = torch.empty(B, KV, T, hd, dtype=torch.bfloat16, device=x.device)
    v = torch.empty(B, KV, T, hd, dtype=torch.bfloat16, device=x.device)
    st = attn_qkv_proj_fwd(x.data_ptr(), w_qkv.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, D, H, KV,
                           hd, pos0, rope_base, _dtype_code(x), _stream_ptr(stream))
    _check(st)
    return q, k, v


def qkv_proj_cache(x, w_qkv, k_cache, v_cache, cache_lens, H, *, rope_base=10000.0, stream=None):
    """attn_qkv_proj_cache_fwd: k/v of the T new tokens go to slots cache_lens[b] + t. Returns q."""
    import torch

    _require({"x": x, "w_qkv": w_qkv, "k_cache": k_cache, "v_cache": v_cache})
    _require({"cache_lens": cache_lens}, dtype=torch.int32)
    B, T, D = x.shape
    KV, Lmax, hd = k_cache.shape[1], k_cache.shape[2], k_cache.shape[3]
    for n_, t_, shp in (("w_qkv", w_qkv, ((H + 2 * KV) * hd, D)), ("v_cache", v_cache, (B, KV, Lmax, hd)),
                        ("k_cache", k_cache, (B, KV, Lmax, hd)), ("cache_lens", cache_lens, (B,))):
        _require_shape(n_, t_, shp)
    _require_gpu(x, w_qkv, k_cache, v_cache, cache_lens)
    q = torch.empty(B, H, T, hd, dtype=torch.bfloat16, device=x.device)
    st = attn_qkv_proj_cache_fwd(x.data_ptr(), w_qkv.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                 cache_lens.data_ptr(), B, T, D, H, KV, hd, Lmax, rope_base, _dtype_code(x),
                                 _stream_ptr(stream))
    _check(st)
    return q


def out_proj(o, w_o, *, out_dtype=None, stream=None):
    """attn_out_proj_fwd on GPU tensors o [B,H,T,hd] bf16, w_o [D, H*hd] bf16. Returns y [B,T,D]."""
    import torch

    _require({"o": o, "w_o": w_o})
    B, H, T, hd = o.shape
    D = w_o.shape[0]
    _require_shape("w_o", w_o, (D, H * hd))
    _require_gpu(o, w_o)
    y = torch.empty(B, T, D, dtype=torch.bfloat16 if out_dtype is None else out_dtype, device=o.device)
    st = attn_out_proj_fwd(o.data_ptr(), w_o.data_ptr(), y.data_ptr(), B, T, H, hd, D, _dtype_code(o), _dtype_code(y),
                           _stream_ptr(stream))
    _check(st)
    return y
