"""The torch helpers of the binding refuse tensors whose raw pointers would be
misread by the library (strided views, mismatched dtypes, host memory, wrong
shapes) before any launch. Runs on the CPU: every case raises before the first
call into libattn.so."""
import pytest
import torch

from transformer_attention_02_amd import binding as bd

bf = torch.bfloat16


def dec_inputs(B=2, H=8, KV=2, hd=64, Lmax=40, dtype=bf):
    return dict(q=torch.zeros(B, H, hd, dtype=dtype), k_new=torch.zeros(B, KV, hd, dtype=dtype),
                v_new=torch.zeros(B, KV, hd, dtype=dtype), k_cache=torch.zeros(B, KV, Lmax, hd, dtype=dtype),
                v_cache=torch.zeros(B, KV, Lmax, hd, dtype=dtype), cache_lens=torch.zeros(B, dtype=torch.int32))


def call_decode(d, **kw):
    return bd.decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["cache_lens"], **kw)


def test_decode_refuses_a_strided_cache_view():
    d = dec_inputs(Lmax=80)
    d["k_cache"] = d["k_cache"][:, :, :40]      # a view into a longer cache: rows of the parent buffer
    d["v_cache"] = d["v_cache"][:, :, :40]
    with pytest.raises(ValueError, match="contiguous"):
        call_decode(d)


def test_decode_refuses_mismatched_dtypes():
    d = dec_inputs()
    d["k_cache"] = d["k_cache"].float()
    with pytest.raises(TypeError, match="k_cache"):
        call_decode(d)
    d = dec_inputs()
    d["cache_lens"] = d["cache_lens"].long()
    with pytest.raises(TypeError, match="cache_lens"):
        call_decode(d)


def test_decode_refuses_host_tensors_and_half_an_append():
    d = dec_inputs()
    with pytest.raises(ValueError, match="GPU tensor"):
        call_decode(d)
    d["v_new"] = None
    with pytest.raises(ValueError, match="both"):
        call_decode(d)


def test_decode_refuses_wrong_shapes():
    d = dec_inputs()
    d["v_cache"] = torch.zeros(2, 2, 41, 64, dtype=bf)
    with pytest.raises(ValueError, match="v_cache"):
        call_decode(d)


def test_decode_fp8_needs_uint8_caches():
    d = dec_inputs()
    with pytest.raises(TypeError, match="uint8"):
        bd.decode_fp8(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["cache_lens"], 1.0, 1.0)


def test_prefill_refuses_bad_tensors():
    q = torch.zeros(1, 4, 16, 64, dtype=bf)
    k = torch.zeros(1, 2, 16, 64, dtype=bf)
    with pytest.raises(ValueError, match="contiguous"):
        bd.prefill(q.transpose(2, 3), k, k)
    with pytest.raises(TypeError, match="v"):
        bd.prefill(q, k, k.float())
    with pytest.raises(ValueError, match="GPU tensor"):
        bd.prefill(q, k, k)


def test_backward_refuses_mismatched_dout():
    q = torch.zeros(1, 4, 16, 64, dtype=bf)
    k = torch.zeros(1, 2, 16, 64, dtype=bf)
    out = torch.zeros(1, 4, 16, 64, dtype=bf)
    lse = torch.zeros(1, 4, 16)
    with pytest.raises(TypeError, match="dout"):
        bd.prefill_bwd(q, k, k, out, lse, out.float())
    with pytest.raises(TypeError, match="lse"):
        bd.prefill_bwd(q, k, k, out, lse.double(), out)


def test_latent_and_projection_helpers_check_their_operands():
    q = torch.zeros(2, 4, 64, dtype=bf)
    c_new = torch.zeros(2, 256, dtype=bf)
    c_cache = torch.zeros(2, 30, 256, dtype=bf)
    w = torch.zeros(4, 256, 64, dtype=bf)
    lens = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(TypeError, match="w_uv"):
        bd.decode_latent(q, c_new, c_cache, lens, w, w.float())
    with pytest.raises(ValueError, match="c_cache"):
        bd.decode_latent(q, c_new, c_cache[:, ::2], lens, w, w)
    x = torch.zeros(1, 8, 128, dtype=bf)
    wq = torch.zeros((4 + 2 * 2) * 64, 128, dtype=bf)
    with pytest.raises(TypeError, match="w_qkv"):
        bd.qkv_proj(x, wq.float(), 4, 2)
    with pytest.raises(ValueError, match="contiguous"):
        bd.out_proj(torch.zeros(1, 4, 8, 64, dtype=bf).transpose(1, 2), torch.zeros(128, 256, dtype=bf))
