"""Causal multi-head scaled dot-product self-attention for MI355X (gfx950).

Thin Python binding over the C ABI of `libgattn.so` (declared in
include/gattn.h).  Every step of the computation runs in the library's HIP
kernels; this module only checks tensors and passes device pointers, sizes and
torch's current HIP stream.  There is no fallback: if the library is missing
or fails to load, importing the binding raises.

Low-level names mirror the C ABI (`gattn_fwd`, `gattn_bwd`, ...) and take
preallocated torch tensors.  `attention_forward` / `attention_backward`
allocate the outputs with torch and call those; `attention_forward_qkv` /
`attention_backward_qkv` do the same for a GPT block's fused (B, T, 3C)
projection output, reading q, k, v in place and writing y (B, T, C) and the
gradient dqkv (B, T, 3C) through the strided entry points.
`attention_forward_dropout` / `attention_backward_dropout` add dropout on the
attention weights (mask from a seed and an offset; with return_keep the
forward also returns its keep decisions as bits, which the backward then
reads instead of drawing them again).
"""
from ._binding import (  # noqa: F401
    BF16,
    F16,
    F32,
    GattnError,
    attention_backward,
    attention_backward_dropout,
    attention_backward_qkv,
    attention_decode,
    attention_forward,
    attention_forward_dropout,
    attention_forward_qkv,
    gattn_bwd,
    gattn_bwd_dropout,
    gattn_bwd_dropout_workspace_bytes,
    gattn_bwd_dkdv,
    gattn_bwd_dq,
    gattn_bwd_noalloc,
    gattn_bwd_noalloc_max_bytes,
    gattn_bwd_preprocess,
    gattn_bwd_strided,
    gattn_bwd_workspace_bytes,
    gattn_fwd,
    gattn_fwd_decode,
    gattn_dropout_keep_bytes,
    gattn_dropout_mask,
    gattn_fwd_decode_workspace_bytes,
    gattn_fwd_dropout,
    gattn_fwd_strided,
    gattn_status_string,
    library_path,
    load_library,
)
