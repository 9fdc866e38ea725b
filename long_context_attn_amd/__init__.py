"""Lightning Attention (MiniMax-01 linear-attention layer) on AMD MI355X.

    from long_context_attn_amd import prefill, prefill_varlen, state, backward, decode

The compute path is liblightning_attn.so (hand-written HIP kernels for
gfx950, C ABI in include/lightning_attn.h); this package only marshals torch
tensors into it.  There is no CPU fallback: if the library is not built the
calls raise.
"""
from .ops import (LightningAttnDeviceError, LightningAttnError, backward,  # noqa: F401
                  backward_varlen,
                  backward_workspace_size, decode, decode_noalloc, decode_workspace_size,
                  layer_prefill,
                  layer_workspace_size, library, prefill, prefill_varlen, prefill_workspace_size,
                  saved_size, softmax_decode, softmax_decode_workspace_size, softmax_prefill,
                  softmax_prefill_varlen, softmax_workspace_size, state,
                  state_varlen, state_workspace_size, status_string, workspace_status)

__all__ = ["prefill", "prefill_varlen", "state", "state_varlen", "backward", "backward_varlen",
           "layer_prefill", "decode", "decode_noalloc", "prefill_workspace_size", "state_workspace_size",
           "backward_workspace_size", "layer_workspace_size", "decode_workspace_size", "library",
           "saved_size",
           "softmax_prefill", "softmax_prefill_varlen", "softmax_workspace_size",
           "softmax_decode", "softmax_decode_workspace_size",
           "status_string", "workspace_status", "LightningAttnError", "LightningAttnDeviceError"]
