"""Python binding of liblightning_attn.so (ctypes; argument marshalling only).

Every step of the layer runs in the library's HIP kernels; torch is used for
device memory and the current stream.  The calls mirror the C ABI declared in
include/lightning_attn.h:

    prefill(q, k, v, gate, weight, ...)            q: [B, N, H, D]
    prefill_varlen(q, k, v, gate, weight, cu, ...) q: [T, H, D], cu: int32 [nseq+1]
    state(k, v, ...) / state_varlen(k, v, cu, ...) final states only, [nseq, H, D, D]
    backward(q, k, v, gate, weight, dout, ...)     gradients of a prefill (and _varlen)
    layer_prefill(x, w_qkvg, weight, w_out, ...)   projections + attention, x: [B, N, hidden]
    decode(q, k, v, gate, weight, state, ...)      q: [S, H, D], state updated in place

The layer is the Lightning Attention Mechanism of "Diving into MiniMax01 405B
MoE" (section "Hybrid Modeling"): SiLU on q/k/v, causal Y = Q (K^T V) against
a running fp32 state, then RMSNorm(Y) * sigmoid(gate).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblightning_attn.so")

LA_DTYPE = {torch.float32: 0, torch.bfloat16: 1}
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t


class LightningAttnError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__("lightning_attn: %s (status %d)" % (text, status))
        self.status = status


def library():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("%s is missing: build it with `python -m long_context_attn_amd.build`"
                               % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        lib.lightning_attn_status_string.argtypes = [_I]
        lib.lightning_attn_status_string.restype = ctypes.c_char_p
        lib.lightning_attn_workspace_status.argtypes = [_P, _SZ, ctypes.POINTER(ctypes.c_int32),
                                                        _P]
        lib.lightning_attn_workspace_status.restype = _I
        lib.lightning_attn_prefill_workspace_size.argtypes = [_I64, _I, _I, _I, _I, _I, _I]
        lib.lightning_attn_prefill_workspace_size.restype = _SZ
        lib.lightning_attn_prefill.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I64, _I, _I,
                                               _I, _I, _F, _I, _P, _SZ, _P]
        lib.lightning_attn_prefill.restype = _I
        lib.lightning_attn_prefill_varlen.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I64, _P,
                                                      _P, _I, _I, _I, _I, _F, _I, _P, _SZ, _P]
        lib.lightning_attn_prefill_varlen.restype = _I
        lib.lightning_attn_state_workspace_size.argtypes = [_I64, _I, _I, _I, _I, _I, _I]
        lib.lightning_attn_state_workspace_size.restype = _SZ
        lib.lightning_attn_state.argtypes = [_P, _P, _P, _P, _I, _I64, _I, _I, _I, _I, _I, _P, _SZ,
                                             _P]
        lib.lightning_attn_state.restype = _I
        lib.lightning_attn_state_varlen.argtypes = [_P, _P, _P, _I, _I64, _P, _P, _I, _I, _I, _I,
                                                    _I, _P, _SZ, _P]
        lib.lightning_attn_state_varlen.restype = _I
        lib.lightning_attn_backward_workspace_size.argtypes = [_I64, _I, _I, _I, _I, _I, _I]
        lib.lightning_attn_backward_workspace_size.restype = _SZ
        lib.lightning_attn_backward.argtypes = [_P] * 14 + [_I, _I64, _I, _I, _I, _I, _F, _I, _P,
                                                            _SZ, _P]
        lib.lightning_attn_backward.restype = _I
        lib.lightning_attn_backward_varlen.argtypes = ([_P] * 7 + [_I, _I64] + [_P] * 8 +
                                                       [_I, _I, _I, _I, _F, _I, _P, _SZ, _P])
        lib.lightning_attn_backward_varlen.restype = _I
        lib.lightning_attn_saved_size.argtypes = [_I64, _I, _I, _I, _I, _I, _I]
        lib.lightning_attn_saved_size.restype = _SZ
        lib.lightning_attn_prefill_save.argtypes = [_P] * 8 + [_I, _I64, _I, _I, _I, _I, _F, _I,
                                                               _P, _SZ, _P, _SZ, _P]
        lib.lightning_attn_prefill_save.restype = _I
        lib.lightning_attn_prefill_varlen_save.argtypes = ([_P] * 7 + [_I, _I64, _P, _P] +
                                                           [_I, _I, _I, _I, _F, _I, _P, _SZ, _P,
                                                            _SZ, _P])
        lib.lightning_attn_prefill_varlen_save.restype = _I
        lib.lightning_attn_backward_saved.argtypes = ([_P] * 14 + [_I, _I64, _I, _I, _I, _I, _F,
                                                                   _I, _P, _SZ, _P, _SZ, _P])
        lib.lightning_attn_backward_saved.restype = _I
        lib.lightning_attn_backward_varlen_saved.argtypes = ([_P] * 7 + [_I, _I64] + [_P] * 8 +
                                                             [_I, _I, _I, _I, _F, _I, _P, _SZ, _P,
                                                              _SZ, _P])
        lib.lightning_attn_backward_varlen_saved.restype = _I
        lib.lightning_attn_layer_workspace_size.argtypes = [_I64, _I, _I, _I, _I]
        lib.lightning_attn_layer_workspace_size.restype = _SZ
        lib.lightning_attn_layer_prefill.argtypes = [_P] * 7 + [_I, _I64, _I, _I, _I, _I, _F, _P,
                                                                _SZ, _P]
        lib.lightning_attn_layer_prefill.restype = _I
        lib.lightning_attn_softmax_workspace_size.argtypes = [_I64, _I, _I, _I, _I]
        lib.lightning_attn_softmax_workspace_size.restype = _SZ
        _D = ctypes.c_double
        lib.lightning_attn_softmax_prefill.argtypes = [_P] * 4 + [_I, _I64, _I, _I, _I, _D, _F, _I,
                                                                 _P, _SZ, _P]
        lib.lightning_attn_softmax_prefill.restype = _I
        lib.lightning_attn_softmax_prefill_varlen.argtypes = [_P] * 5 + [_I, _I64, _I, _I, _I, _D,
                                                                        _F, _I, _P, _SZ, _P]
        lib.lightning_attn_softmax_prefill_varlen.restype = _I
        lib.lightning_attn_softmax_decode_workspace_size.argtypes = [_I, _I, _I, _I]
        lib.lightning_attn_softmax_decode_workspace_size.restype = _SZ
        lib.lightning_attn_softmax_decode.argtypes = [_P] * 7 + [_I, _I, _I, _I, _I, _D, _F, _I,
                                                                _P, _SZ, _P]
        lib.lightning_attn_softmax_decode.restype = _I
        lib.lightning_attn_decode_workspace_size.argtypes = [_I, _I, _I]
        lib.lightning_attn_decode_workspace_size.restype = _SZ
        lib.lightning_attn_decode.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _F, _I, _P,
                                              _SZ, _P]
        lib.lightning_attn_decode.restype = _I
        lib.lightning_attn_decode_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _F,
                                                      _I, _P]
        lib.lightning_attn_decode_noalloc.restype = _I
        _lib = lib
    return _lib


class LightningAttnDeviceError(RuntimeError):
    """A condition the kernels recorded in the workspace (the call itself had
    returned ok): 1 = cu_seqlens inconsistent, 2 = chunk table overflow, 3 = a
    cross-workgroup wait of the fused walk gave up."""

    TEXT = {1: "cu_seqlens is inconsistent (cu[0] != 0, a decreasing entry, or cu[nseq] != "
               "total_tokens); nothing was processed",
            2: "chunk table overflow",
            3: "a cross-workgroup wait of the fused prefill walk gave up (the workgroups of "
               "one chunk could not all run at once)"}

    def __init__(self, status):
        self.error, self.site, self.chunk, self.head = status
        text = self.TEXT.get(self.error, "unknown device error")
        if self.error == 3:
            text += " (wait site %d, chunk %d, head %d)" % (self.site, self.chunk, self.head)
        super().__init__("lightning_attn: %s (device error %d); the outputs are unspecified"
                         % (text, self.error))


def status_string(status: int) -> str:
    return library().lightning_attn_status_string(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise LightningAttnError(status, status_string(status))


def workspace_status(workspace: torch.Tensor):
    """Device-side status of the last call that used `workspace` (waits for the
    current stream): (error, wait site, chunk, head), all 0 when ok."""
    out = (ctypes.c_int32 * 4)()
    _check(library().lightning_attn_workspace_status(
        _ptr(workspace), workspace.numel() * workspace.element_size(), out,
        _stream(workspace.device)))
    return tuple(int(x) for x in out)


def _debug_default(check):
    if check is None:
        return os.environ.get("LA_DEBUG", "0") not in ("", "0")
    return bool(check)


def _check_device(workspace, check):
    """With check (or LA_DEBUG=1 in the environment): wait for the call and raise
    LightningAttnDeviceError if the kernels recorded an error."""
    if _debug_default(check):
        st = workspace_status(workspace)
        if st[0] != 0:
            raise LightningAttnDeviceError(st)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in LA_DTYPE:
        raise TypeError("lightning_attn supports float32 and bfloat16 activations, got %s" % t.dtype)
    return LA_DTYPE[t.dtype]


def _same(ref: torch.Tensor, *ts):
    for t in ts:
        if t.dtype != ref.dtype or t.device != ref.device:
            raise TypeError("all activations and the norm weight must share dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _state(t, shape, device, name):
    if t is None:
        return None
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous() \
            or t.device != device:
        raise ValueError("%s must be a contiguous float32 tensor of shape %s on %s"
                         % (name, tuple(shape), device))
    return t


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def prefill_workspace_size(total_tokens, nseq, heads, head_dim, block=64, chunk_tokens=0,
                           dtype=torch.bfloat16) -> int:
    return int(library().lightning_attn_prefill_workspace_size(
        int(total_tokens), int(nseq), int(heads), int(head_dim), int(block), int(chunk_tokens),
        LA_DTYPE[dtype]))


def decode_workspace_size(nseq, heads, head_dim) -> int:
    return int(library().lightning_attn_decode_workspace_size(int(nseq), int(heads), int(head_dim)))


def _workspace(nbytes, device, given):
    if given is not None:
        if given.numel() * given.element_size() < nbytes:
            raise ValueError("workspace too small: need %d bytes" % nbytes)
        return given
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def saved_size(total_tokens, nseq, heads, head_dim, block=64, chunk_tokens=0,
               dtype=torch.bfloat16) -> int:
    """Bytes of the activations a prefill saves for its backward (0 where the
    path does not save: only bf16, head_dim 128, block 64)."""
    return int(library().lightning_attn_saved_size(
        int(total_tokens), int(nseq), int(heads), int(head_dim), int(block), int(chunk_tokens),
        LA_DTYPE[dtype]))


def _saved_buffer(nbytes, device, given):
    if nbytes == 0:
        raise LightningAttnError(3, status_string(3))
    return _workspace(nbytes, device, given)


def prefill(q, k, v, gate, weight, *, block=64, eps=1e-6, initial_state=None,
            return_final_state=False, chunk_tokens=0, out=None, final_state=None,
            workspace=None, check=None, save_for_backward=False, saved=None):
    """Causal Lightning Attention prefill of B rows of N tokens.

    q, k, v, gate: [B, N, H, D] (float32 or bfloat16, contiguous, one device);
    weight: [H*D]; initial_state: [B, H, D, D] float32 or None (zeros).
    Returns out [B, N, H, D] (and the final state [B, H, D, D] if requested).
    With save_for_backward, also returns (last) the saved activations (a uint8
    tensor, or `saved` filled in place) for backward(..., saved=...).
    """
    _same(q, k, v, gate, weight)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape or gate.shape != q.shape:
        raise ValueError("q, k, v, gate must share one [B, N, H, D] shape")
    B, N, H, D = q.shape
    if weight.numel() != H * D:
        raise ValueError("weight must have H*D elements")
    dev = q.device
    init = _state(initial_state, (B, H, D, D), dev, "initial_state")
    if out is None:
        out = torch.empty_like(q)
    fs = None
    if return_final_state:
        fs = final_state if final_state is not None else torch.empty(B, H, D, D, dtype=torch.float32,
                                                                    device=dev)
        _state(fs, (B, H, D, D), dev, "final_state")
    ws_bytes = prefill_workspace_size(B * N, B, H, D, block, chunk_tokens, q.dtype)
    if ws_bytes == 0:
        raise LightningAttnError(3, status_string(3))
    ws = _workspace(ws_bytes, dev, workspace)
    if save_for_backward:
        sv_bytes = saved_size(B * N, B, H, D, block, chunk_tokens, q.dtype)
        sv = _saved_buffer(sv_bytes, dev, saved)
        _check(library().lightning_attn_prefill_save(
            _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(weight), _ptr(out), _ptr(init), _ptr(fs),
            B, N, H, D, int(block), int(chunk_tokens), float(eps), _dtype(q), _ptr(sv), sv_bytes,
            _ptr(ws), ws_bytes, _stream(dev)))
    else:
        _check(library().lightning_attn_prefill(
            _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(weight), _ptr(out), _ptr(init), _ptr(fs),
            B, N, H, D, int(block), int(chunk_tokens), float(eps), _dtype(q), _ptr(ws), ws_bytes,
            _stream(dev)))
    _check_device(ws, check)
    res = (out, fs) if return_final_state else (out,)
    if save_for_backward:
        res = res + (sv,)
    return res if len(res) > 1 else res[0]


def prefill_varlen(q, k, v, gate, weight, cu_seqlens, *, block=64, eps=1e-6, initial_state=None,
                   return_final_state=False, chunk_tokens=0, out=None, final_state=None,
                   workspace=None, check=None, save_for_backward=False, saved=None):
    """Causal prefill of sequences packed back to back.

    q, k, v, gate: [T, H, D]; cu_seqlens: int32 [nseq+1] on the same device
    (0 = cu[0] <= ... <= cu[nseq] = T); initial_state: [nseq, H, D, D] or None.
    save_for_backward / saved: as for `prefill`.
    """
    _same(q, k, v, gate, weight)
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape or gate.shape != q.shape:
        raise ValueError("q, k, v, gate must share one [T, H, D] shape")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != q.device \
            or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector on the activations' device")
    T, H, D = q.shape
    nseq = cu_seqlens.numel() - 1
    if nseq < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    if weight.numel() != H * D:
        raise ValueError("weight must have H*D elements")
    dev = q.device
    init = _state(initial_state, (nseq, H, D, D), dev, "initial_state")
    if out is None:
        out = torch.empty_like(q)
    fs = None
    if return_final_state:
        fs = final_state if final_state is not None else torch.empty(nseq, H, D, D,
                                                                    dtype=torch.float32, device=dev)
        _state(fs, (nseq, H, D, D), dev, "final_state")
    ws_bytes = prefill_workspace_size(T, nseq, H, D, block, chunk_tokens, q.dtype)
    if ws_bytes == 0:
        raise LightningAttnError(3, status_string(3))
    ws = _workspace(ws_bytes, dev, workspace)
    if save_for_backward:
        sv_bytes = saved_size(T, nseq, H, D, block, chunk_tokens, q.dtype)
        sv = _saved_buffer(sv_bytes, dev, saved)
        _check(library().lightning_attn_prefill_varlen_save(
            _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(weight), _ptr(out), _ptr(cu_seqlens),
            nseq, T, _ptr(init), _ptr(fs), H, D, int(block), int(chunk_tokens), float(eps),
            _dtype(q), _ptr(sv), sv_bytes, _ptr(ws), ws_bytes, _stream(dev)))
    else:
        _check(library().lightning_attn_prefill_varlen(
            _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(weight), _ptr(out), _ptr(cu_seqlens),
            nseq, T, _ptr(init), _ptr(fs), H, D, int(block), int(chunk_tokens), float(eps),
            _dtype(q), _ptr(ws), ws_bytes, _stream(dev)))
    _check_device(ws, check)
    res = (out, fs) if return_final_state else (out,)
    if save_for_backward:
        res = res + (sv,)
    return res if len(res) > 1 else res[0]


def state_workspace_size(total_tokens, nseq, heads, head_dim, block=64, chunk_tokens=0,
                         dtype=torch.bfloat16) -> int:
    return int(library().lightning_attn_state_workspace_size(
        int(total_tokens), int(nseq), int(heads), int(head_dim), int(block), int(chunk_tokens),
        LA_DTYPE[dtype]))


def state(k, v, *, block=64, initial_state=None, final_state=None, chunk_tokens=0,
          workspace=None, check=None):
    """Final states of B rows of N tokens without outputs: initial_state (or zeros)
    + sum_t SiLU(k_t)^T SiLU(v_t).  k, v: [B, N, H, D]; returns [B, H, D, D] fp32."""
    _same(k, v)
    if k.dim() != 4 or v.shape != k.shape:
        raise ValueError("k, v must share one [B, N, H, D] shape")
    B, N, H, D = k.shape
    dev = k.device
    init = _state(initial_state, (B, H, D, D), dev, "initial_state")
    fs = final_state if final_state is not None else torch.empty(B, H, D, D, dtype=torch.float32,
                                                                device=dev)
    _state(fs, (B, H, D, D), dev, "final_state")
    ws_bytes = state_workspace_size(B * N, B, H, D, block, chunk_tokens, k.dtype)
    if ws_bytes == 0:
        raise LightningAttnError(3, status_string(3))
    ws = _workspace(ws_bytes, dev, workspace)
    _check(library().lightning_attn_state(
        _ptr(k), _ptr(v), _ptr(init), _ptr(fs), B, N, H, D, int(block), int(chunk_tokens),
        _dtype(k), _ptr(ws), ws_bytes, _stream(dev)))
    _check_device(ws, check)
    return fs


def state_varlen(k, v, cu_seqlens, *, block=64, initial_state=None, final_state=None,
                 chunk_tokens=0, workspace=None, check=None):
    """Final states of packed sequences without outputs.  k, v: [T, H, D];
    cu_seqlens: int32 [nseq+1] on the same device; returns [nseq, H, D, D] fp32."""
    _same(k, v)
    if k.dim() != 3 or v.shape != k.shape:
        raise ValueError("k, v must share one [T, H, D] shape")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != k.device \
            or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector on the activations' device")
    T, H, D = k.shape
    nseq = cu_seqlens.numel() - 1
    if nseq < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    dev = k.device
    init = _state(initial_state, (nseq, H, D, D), dev, "initial_state")
    fs = final_state if final_state is not None else torch.empty(nseq, H, D, D,
                                                                dtype=torch.float32, device=dev)
    _state(fs, (nseq, H, D, D), dev, "final_state")
    ws_bytes = state_workspace_size(T, nseq, H, D, block, chunk_tokens, k.dtype)
    if ws_bytes == 0:
        raise LightningAttnError(3, status_string(3))
    ws = _workspace(ws_bytes, dev, workspace)
    _check(library().lightning_attn_state_varlen(
        _ptr(k), _ptr(v), _ptr(cu_seqlens), nseq, T, _ptr(init), _ptr(fs), H, D, int(block),
        int(chunk_tokens), _dtype(k), _ptr(ws), ws_bytes, _stream(dev)))
    _check_device(ws, check)
    return fs


def backward_workspace_size(total_tokens, nseq, heads, head_dim, block=64, chunk_tokens=0,
                            dtype=torch.bfloat16) -> int:
    return int(library().lightning_attn_backward_workspace_size(
        int(total_tokens), int(nseq), int(heads), int(head_dim), int(block), int(chunk_tokens),
        LA_DTYPE[dtype]))


def _backward_outputs(q, nseq, H, D, want_d_init):
    dev = q.device
    grads = [torch.empty_like(q) for _ in range(4)]
    dw = torch.empty(H * D, dtype=torch.float32, device=dev)
    d_init = torch.empty(nseq, H, D, D, dtype=torch.float32, device=dev) if want_d_init else None
    return grads, dw, d_init


def _saved_arg(saved, nbytes, device):
    if not isinstance(saved, torch.Tensor) or saved.dtype != torch.uint8 or \
            not saved.is_contiguous() or saved.device != device:
        raise ValueError("saved must be the uint8 tensor a prefill with save_for_backward returned "
                         "(contiguous, on the activations' device)")
    if nbytes == 0:
        raise LightningAttnError(3, status_string(3))
    if saved.numel() < nbytes:
        raise ValueError("saved too small: need %d bytes" % nbytes)
    return saved, saved.numel()


def backward(q, k, v, gate, weight, dout, *, block=64, eps=1e-6, initial_state=None,
             d_final_state=None, return_d_initial_state=False, chunk_tokens=0, workspace=None,
             check=None, saved=None):
    """Gradients of `prefill` for a loss with gradient `dout` w.r.t. the output (and
    `d_final_state` w.r.t. the final states).  q, k, v, gate, dout: [B, N, H, D].
    Returns (dq, dk, dv, dgate, dweight, d_initial_state or None); dweight and
    d_initial_state are float32.  saved: the activations `prefill(...,
    save_for_backward=True)` returned for the same inputs (y and the chunk
    states are then read instead of recomputed)."""
    _same(q, q, k, v, gate, weight, dout)
    if q.dim() != 4 or any(t.shape != q.shape for t in (k, v, gate, dout)):
        raise ValueError("q, k, v, gate, dout must share one [B, N, H, D] shape")
    B, N, H, D = q.shape
    if weight.numel() != H * D:
        raise ValueError("weight must have H*D elements")
    dev = q.device
    init = _state(initial_state, (B, H, D, D), dev, "initial_state")
    dfin = _state(d_final_state, (B, H, D, D), dev, "d_final_state")
    (dq, dk, dv, dg), dw, d_init = _backward_outputs(q, B, H, D, return_d_initial_state)
    ws_bytes = backward_workspace_size(B * N, B, H, D, block, chunk_tokens, q.dtype)
    if ws_bytes == 0:
        raise LightningAttnError(3, status_string(3))
    ws = _workspace(ws_bytes, dev, workspace)
    if saved is not None:
        sv, sv_bytes = _saved_arg(saved, saved_size(B * N, B, H, D, block, chunk_tokens, q.dtype),
                                 dev)
        _check(library().lightning_attn_backward_saved(
            _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(weight), _ptr(dout), _ptr(init),
            _ptr(dfin), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dw), _ptr(d_init), B, N, H,
            D, int(block), int(chunk_tokens), float(eps), _dtype(q), _ptr(sv), sv_bytes, _ptr(ws),
            ws_bytes, _stream(dev)))
    else:
        _check(library().lightning_attn_backward(
            _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(weight), _ptr(dout), _ptr(init),
            _ptr(dfin), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dw), _ptr(d_init), B, N, H,
            D, int(block), int(chunk_tokens), float(eps), _dtype(q), _ptr(ws), ws_bytes,
            _stream(dev)))
    _check_device(ws, check)
    return dq, dk, dv, dg, dw, d_init


def backward_varlen(q, k, v, gate, weight, dout, cu_seqlens, *, block=64, eps=1e-6,
                    initial_state=None, d_final_state=None, return_d_initial_state=False,
                    chunk_tokens=0, workspace=None, check=None, saved=None):
    """Gradients of `prefill_varlen`; q, k, v, gate, dout: [T, H, D], cu_seqlens int32.
    saved: as for `backward`."""
    _same(q, q, k, v, gate, weight, dout)
    if q.dim() != 3 or any(t.shape != q.shape for t in (k, v, gate, dout)):
        raise ValueError("q, k, v, gate, dout must share one [T, H, D] shape")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != q.device \
            or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector on the activations' device")
    T, H, D = q.shape
    nseq = cu_seqlens.numel() - 1
    if nseq < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    if weight.numel() != H * D:
        raise ValueError("weight must have H*D elements")
    dev = q.device
    init = _state(initial_state, (nseq, H, D, D), dev, "initial_state")
    dfin = _state(d_final_state, (nseq, H, D, D), dev, "d_final_state")
    (dq, dk, dv, dg), dw, d_init = _backward_outputs(q, nseq, H, D, return_d_initial_state)
    ws_bytes = backward_workspace_size(T, nseq, H, D, block, chunk_tokens, q.dtype)
    if ws_bytes == 0:
        raise LightningAttnError(3, status_string(3))
    ws = _workspace(ws_bytes, dev, workspace)
    if saved is not None:
        sv, sv_bytes = _saved_arg(saved, saved_size(T, nseq, H, D, block, chunk_tokens, q.dtype), dev)
        _check(library().lightning_attn_backward_varlen_saved(
            _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(weight), _ptr(dout), _ptr(cu_seqlens),
            nseq, T, _ptr(init), _ptr(dfin), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dw),
            _ptr(d_init), H, D, int(block), int(chunk_tokens), float(eps), _dtype(q), _ptr(sv),
            sv_bytes, _ptr(ws), ws_bytes, _stream(dev)))
    else:
        _check(library().lightning_attn_backward_varlen(
            _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(weight), _ptr(dout), _ptr(cu_seqlens),
            nseq, T, _ptr(init), _ptr(dfin), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dw),
            _ptr(d_init), H, D, int(block), int(chunk_tokens), float(eps), _dtype(q), _ptr(ws),
            ws_bytes, _stream(dev)))
    _check_device(ws, check)
    return dq, dk, dv, dg, dw, d_init


def layer_workspace_size(total_tokens, nseq, hidden, heads, head_dim=128) -> int:
    return int(library().lightning_attn_layer_workspace_size(
        int(total_tokens), int(nseq), int(hidden), int(heads), int(head_dim)))


GEMM_BACKENDS = {"mfma": 0, "hipblaslt": 1}


def layer_prefill(x, w_qkvg, weight, w_out, *, eps=1e-6, initial_state=None,
                  return_final_state=False, out=None, final_state=None, workspace=None,
                  check=None, gemm="mfma"):
    """The layer with its projections.  x: [B, N, hidden] bf16; w_qkvg: [4, hidden, H*D]
    (Wq, Wk, Wv, Wg, y = x W); weight: [H*D]; w_out: [H*D, hidden].  Head dim 128.
    gemm: "mfma" (the library's GEMM kernel, hidden % 64 == 0) or "hipblaslt"."""
    if gemm not in GEMM_BACKENDS:
        raise ValueError("gemm must be one of %s" % sorted(GEMM_BACKENDS))
    _same(x, x, w_qkvg, weight, w_out)
    if x.dim() != 3 or w_qkvg.dim() != 3 or w_qkvg.shape[0] != 4 or w_qkvg.shape[1] != x.shape[2]:
        raise ValueError("x must be [B, N, hidden] and w_qkvg [4, hidden, H*D]")
    B, N, hidden = x.shape
    HD = w_qkvg.shape[2]
    D = 128
    if HD % D != 0 or weight.numel() != HD or tuple(w_out.shape) != (HD, hidden):
        raise ValueError("weight must be [H*D] and w_out [H*D, hidden], head_dim 128")
    H = HD // D
    dev = x.device
    if out is None:
        out = torch.empty_like(x)
    _same(x, out)
    init = _state(initial_state, (B, H, D, D), dev, "initial_state")
    fs = final_state
    if return_final_state and fs is None:
        fs = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    _state(fs, (B, H, D, D), dev, "final_state")
    ws_bytes = layer_workspace_size(B * N, B, hidden, H, D)
    if ws_bytes == 0:
        raise LightningAttnError(3, status_string(3))
    ws = _workspace(ws_bytes, dev, workspace)
    _check(library().lightning_attn_layer_prefill(
        _ptr(x), _ptr(w_qkvg), _ptr(weight), _ptr(w_out), _ptr(out), _ptr(init), _ptr(fs), B, N,
        hidden, H, D, GEMM_BACKENDS[gemm], float(eps), _ptr(ws), ws_bytes, _stream(dev)))
    _check_device(ws, check)
    return (out, fs) if return_final_state else out


def decode(q, k, v, gate, weight, state, *, eps=1e-6, out=None, workspace=None):
    """One decode step for S sequences; `state` [S, H, D, D] fp32 is updated in place."""
    _same(q, k, v, gate, weight)
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape or gate.shape != q.shape:
        raise ValueError("q, k, v, gate must share one [S, H, D] shape")
    S, H, D = q.shape
    if weight.numel() != H * D:
        raise ValueError("weight must have H*D elements")
    dev = q.device
    _state(state, (S, H, D, D), dev, "state")
    if out is None:
        out = torch.empty_like(q)
    ws_bytes = decode_workspace_size(S, H, D)
    ws = _workspace(ws_bytes, dev, workspace)
    _check(library().lightning_attn_decode(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(weight), _ptr(out), _ptr(state), S, H, D,
        float(eps), _dtype(q), _ptr(ws), ws_bytes, _stream(dev)))
    return out


def decode_noalloc(q, k, v, gate, weight, state, *, eps=1e-6, out=None):
    """`decode` through the entry point that allocates nothing: its scratch is
    a fixed array of the library (4 MiB + 64 KiB per GPU); shapes that need
    more raise (status 7).  Calls that overlap on one GPU race.  `out` may be
    passed in so that the call allocates nothing on the torch side either."""
    _same(q, k, v, gate, weight)
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape or gate.shape != q.shape:
        raise ValueError("q, k, v, gate must share one [S, H, D] shape")
    S, H, D = q.shape
    if weight.numel() != H * D:
        raise ValueError("weight must have H*D elements")
    dev = q.device
    _state(state, (S, H, D, D), dev, "state")
    if out is None:
        out = torch.empty_like(q)
    _check(library().lightning_attn_decode_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(weight), _ptr(out), _ptr(state), S, H, D,
        float(eps), _dtype(q), _stream(dev)))
    return out


ROPE_BASE = 1e7  # the model card's rotary base frequency


def softmax_workspace_size(total_tokens, nseq, heads, head_dim=128, rope_dim=64) -> int:
    return int(library().lightning_attn_softmax_workspace_size(
        int(total_tokens), int(nseq), int(heads), int(head_dim), int(rope_dim)))


def _softmax_args(q, k, v, rope_dim, scale):
    _same(q, k, v)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one shape")
    D = q.shape[-1]
    rd = D // 2 if rope_dim is None else int(rope_dim)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    return rd, sc


def softmax_prefill(q, k, v, *, rope_dim=None, rope_base=ROPE_BASE, scale=None, out=None,
                    workspace=None, check=None):
    """The hybrid's softmax attention layer on B rows of N tokens: q and k
    rotated on their first rope_dim features (default head_dim / 2, base 1e7),
    then causal softmax attention with logits scaled by `scale` (default
    1/sqrt(head_dim)).  q, k, v: [B, N, H, D] bf16, D = 128."""
    rd, sc = _softmax_args(q, k, v, rope_dim, scale)
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, N, H, D]")
    B, N, H, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _same(q, out)
    ws_bytes = softmax_workspace_size(B * N, B, H, D, rd)
    if ws_bytes == 0:
        raise LightningAttnError(3, status_string(3))
    ws = _workspace(ws_bytes, q.device, workspace)
    _check(library().lightning_attn_softmax_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, N, H, D, rd, float(rope_base), sc, _dtype(q),
        _ptr(ws), ws_bytes, _stream(q.device)))
    _check_device(ws, check)
    return out


def softmax_prefill_varlen(q, k, v, cu_seqlens, *, rope_dim=None, rope_base=ROPE_BASE, scale=None,
                           out=None, workspace=None, check=None):
    """softmax_prefill on sequences packed back to back: q, k, v [T, H, D] bf16,
    cu_seqlens int32 [nseq+1] on the same device; positions restart at 0 in
    every sequence."""
    rd, sc = _softmax_args(q, k, v, rope_dim, scale)
    if q.dim() != 3:
        raise ValueError("q, k, v must be [T, H, D]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != q.device \
            or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector on the activations' device")
    T, H, D = q.shape
    nseq = cu_seqlens.numel() - 1
    if nseq < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    if out is None:
        out = torch.empty_like(q)
    _same(q, out)
    ws_bytes = softmax_workspace_size(T, nseq, H, D, rd)
    if ws_bytes == 0:
        raise LightningAttnError(3, status_string(3))
    ws = _workspace(ws_bytes, q.device, workspace)
    _check(library().lightning_attn_softmax_prefill_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(cu_seqlens), nseq, T, H, D, rd,
        float(rope_base), sc, _dtype(q), _ptr(ws), ws_bytes, _stream(q.device)))
    _check_device(ws, check)
    return out


def softmax_decode_workspace_size(nseq, max_len, heads, head_dim=128) -> int:
    return int(library().lightning_attn_softmax_decode_workspace_size(
        int(nseq), int(max_len), int(heads), int(head_dim)))


def softmax_decode(q, k, v, k_cache, v_cache, cache_len, *, rope_dim=None, rope_base=ROPE_BASE,
                   scale=None, out=None, workspace=None):
    """One decode step of the softmax layer: q, k, v [S, H, D] bf16 (the new
    token of each sequence); k_cache, v_cache [S, H, max_len, D] bf16 (head-major,
    keys stored rotated), updated in place at slot cache_len[s]; cache_len
    int32 [S] on the device, not advanced here.  Returns out [S, H, D]."""
    rd, sc = _softmax_args(q, k, v, rope_dim, scale)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q, k, v must be [S, H, D] and the caches [S, H, max_len, D]")
    S, H, D = q.shape
    if k_cache.shape[0] != S or k_cache.shape[1] != H or k_cache.shape[3] != D:
        raise ValueError("cache shape does not match q")
    _same(q, k_cache, v_cache)
    if cache_len.dtype != torch.int32 or cache_len.numel() != S or cache_len.device != q.device \
            or not cache_len.is_contiguous():
        raise ValueError("cache_len must be a contiguous int32 vector of S entries on the device")
    max_len = k_cache.shape[2]
    if out is None:
        out = torch.empty_like(q)
    _same(q, out)
    ws_bytes = softmax_decode_workspace_size(S, max_len, H, D)
    if ws_bytes == 0:
        raise LightningAttnError(3, status_string(3))
    ws = _workspace(ws_bytes, q.device, workspace)
    _check(library().lightning_attn_softmax_decode(
        _ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), _ptr(out), S,
        max_len, H, D, rd, float(rope_base), sc, _dtype(q), _ptr(ws), ws_bytes,
        _stream(q.device)))
    return out
