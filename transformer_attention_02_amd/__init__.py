"""MI355X (gfx950) causal grouped-query attention forward: prefill and KV-cache decode.

The compute path is the HIP library ``libattn.so`` built from ``csrc/``; the
Python module :mod:`transformer_attention_02_amd.binding` only marshals
arguments to its C entry points. Importing this package loads nothing; the
library is opened on first use and a missing library is an error.
"""
__all__ = ["binding", "workloads"]
