"""CPU fp64 oracle (test infrastructure only; never used by the product path)."""
from .attention import (  # noqa: F401
    ALIBI_GEOMETRIC,
    ALIBI_NONE,
    ALIBI_PAGE1,
    alibi_slopes,
    apply_rope,
    attention_decode,
    attention_prefill,
    attention_prefill_bwd,
    kv_bytes_per_token,
    prefill_flops,
    rope_inv_freq,
)
from .fp8 import E4M3_MAX, attention_decode_fp8, e4m3_decode, e4m3_encode, e4m3_values  # noqa: F401
from .latent import attention_decode_latent, fold_query  # noqa: F401
from .proj import out_projection, proj_flops, qkv_projection, qkv_projection_to_cache  # noqa: F401
