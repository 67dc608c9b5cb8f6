"""MI355X (gfx950) causal self-attention: forward, backward and KV-cache decode.

The compute lives in libcausal_attn.so (HIP kernels behind the C ABI of include/attn.h);
``binding`` wraps it for PyTorch tensors.  Build it with
``python -m causal_attention_02_amd.build``.
"""
from .binding import (  # noqa: F401
    AttnError,
    AttnOptions,
    attn_bwd,
    attn_decode,
    attn_dropout_mask,
    attn_extend,
    attn_fwd,
    bwd_workspace_bytes,
    decode_workspace,
    device_info,
    dropout_mask_bytes,
    fwd_workspace_bytes,
    lib,
    trace_enable,
    trace_read,
)
