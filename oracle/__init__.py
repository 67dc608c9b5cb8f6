"""fp64 CPU oracle for causal attention -- test infrastructure only (see attn_ref.py)."""
from .attn_ref import (  # noqa: F401
    attention_backward,
    attention_decode,
    attention_extend,
    attention_forward,
    dropout_fields,
    dropout_keep,
    dropout_threshold,
    rms_normalize,
    rope_rotate,
    rope_unrotate,
    segment_starts,
    visible_mask,
)
