"""CPU oracle for the Lightning Attention layer -- test infrastructure only.

Plain fp64 implementation of what the layer computes ("Diving into MiniMax01
405B MoE", section "Hybrid Modeling", Lightning Attention-2 Mechanism steps
1-4).  Only tests/, ``__graft_entry__.smoke()`` and bench.py's cpu_baseline leg
may import this package; the GPU library never does.  It shares no code with
the HIP path: the arithmetic lives in ``la_oracle.c`` (plain C, built with gcc,
no fast-math) and this module only marshals numpy arrays.

It also states the hybrid's other attention, the softmax layer (same page,
"1/8 Softmax Attention"; the model card's Positional Encoding: rotary
embedding on half of the head dimension, base 10,000,000): ``rope`` and
``softmax_attention``.

All functions take numpy arrays of any float dtype and compute in float64
(bf16 and fp32 values convert to float64 exactly).  Layout is token-major:
activations [T, H, D]; states [nseq, H, D, D] with row = key dimension.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB = os.path.join(_HERE, "liblaoracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile la_oracle.c into liblaoracle.so with gcc (IEEE fp64, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    """Open a built oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    lib.la_oracle_prefill.argtypes = [_D, _D, _D, _D, _D, _I64, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_double, _D, _D, _D, _D]
    lib.la_oracle_prefill_blocked.argtypes = [_D, _D, _D, _D, _D, _I64, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_double, _D, _D, _D]
    lib.la_oracle_decode.argtypes = [_D, _D, _D, _D, _D, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_double, _D, _D]
    lib.la_oracle_state.argtypes = [_D, _D, _I64, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, _D]
    lib.la_oracle_backward.argtypes = [_D, _D, _D, _D, _D, _D, _I64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_double, _D, _D,
                                       _D, _D, _D, _D, _D, _D]
    lib.la_oracle_rope.argtypes = [_D, _D, _I64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_double]
    lib.la_oracle_softmax_attention.argtypes = [_D, _D, _D, _I64, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                                ctypes.c_double, _I64, ctypes.c_int64, _D]
    lib.la_oracle_sigmoid.argtypes = [ctypes.c_double]
    lib.la_oracle_sigmoid.restype = ctypes.c_double
    lib.la_oracle_silu.argtypes = [ctypes.c_double]
    lib.la_oracle_silu.restype = ctypes.c_double
    lib.la_oracle_set_threads.argtypes = [ctypes.c_int]
    lib.la_oracle_max_threads.restype = ctypes.c_int
    for f in ("la_oracle_prefill", "la_oracle_prefill_blocked", "la_oracle_decode",
              "la_oracle_state", "la_oracle_backward", "la_oracle_rope",
              "la_oracle_softmax_attention"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _bind(_LIB)
    return _lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (cpu): convert exactly through float64
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(_D)


def _segments(T, cu_seqlens):
    if cu_seqlens is None:
        seg = np.array([0, T], dtype=np.int64)
    else:
        seg = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    if seg[0] != 0 or seg[-1] != T or np.any(np.diff(seg) < 0):
        raise ValueError("segment boundaries must start at 0, be nondecreasing and end at T")
    return seg


def set_threads(n: int) -> None:
    _load().la_oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().la_oracle_max_threads())


def sigmoid(x: float) -> float:
    return float(_load().la_oracle_sigmoid(float(x)))


def silu(x: float) -> float:
    return float(_load().la_oracle_silu(float(x)))


def prefill(q, k, v, g, w, cu_seqlens=None, eps=1e-6, init_state=None, return_y=False,
            return_state=False):
    """Token-recurrence prefill over packed segments.

    q, k, v, g: [T, H, D]; w: [H*D]; cu_seqlens: [nseq+1] segment bounds (None:
    one segment); init_state: [nseq, H, D, D] or None (zeros).
    Returns out [T, H, D] (float64), plus y (pre-norm) and/or final states.
    """
    q, k, v, g, w = (_f64(a) for a in (q, k, v, g, w))
    T, H, D = q.shape
    seg = _segments(T, cu_seqlens)
    nseq = len(seg) - 1
    init = _f64(init_state)
    if init is not None and init.shape != (nseq, H, D, D):
        raise ValueError("init_state shape")
    out = np.empty((T, H, D), np.float64)
    y = np.empty((T, H, D), np.float64) if return_y else None
    fs = np.empty((nseq, H, D, D), np.float64) if return_state else None
    _load().la_oracle_prefill(_p(q), _p(k), _p(v), _p(g), _p(w), seg.ctypes.data_as(_I64), nseq,
                              H, D, float(eps), _p(init), _p(out), _p(y), _p(fs))
    res = (out,) + ((y,) if return_y else ()) + ((fs,) if return_state else ())
    return res[0] if len(res) == 1 else res


def prefill_blocked(q, k, v, g, w, block, cu_seqlens=None, eps=1e-6, init_state=None,
                    return_state=False):
    """Block-tiled prefill (intra-block masked product + inter-block state)."""
    q, k, v, g, w = (_f64(a) for a in (q, k, v, g, w))
    T, H, D = q.shape
    seg = _segments(T, cu_seqlens)
    nseq = len(seg) - 1
    init = _f64(init_state)
    out = np.empty((T, H, D), np.float64)
    fs = np.empty((nseq, H, D, D), np.float64) if return_state else None
    rc = _load().la_oracle_prefill_blocked(_p(q), _p(k), _p(v), _p(g), _p(w),
                                           seg.ctypes.data_as(_I64), nseq, H, D, int(block),
                                           float(eps), _p(init), _p(out), _p(fs))
    if rc != 0:
        raise ValueError("block must be >= 1")
    return (out, fs) if return_state else out


def decode(q, k, v, g, w, state, eps=1e-6):
    """One decode step. q, k, v, g: [S, H, D]; state [S, H, D, D] (not modified).

    Returns (out [S, H, D], new_state [S, H, D, D]) in float64.
    """
    q, k, v, g, w = (_f64(a) for a in (q, k, v, g, w))
    S, H, D = q.shape
    st = _f64(state).copy()
    if st.shape != (S, H, D, D):
        raise ValueError("state shape")
    out = np.empty((S, H, D), np.float64)
    _load().la_oracle_decode(_p(q), _p(k), _p(v), _p(g), _p(w), S, H, D, float(eps), _p(st),
                             _p(out))
    return out, st


def state(k, v, cu_seqlens=None, init_state=None):
    """State after a prefill: S0 + sum_t SiLU(k_t)^T SiLU(v_t) per segment and head."""
    k, v = _f64(k), _f64(v)
    T, H, D = k.shape
    seg = _segments(T, cu_seqlens)
    nseq = len(seg) - 1
    st = np.zeros((nseq, H, D, D), np.float64) if init_state is None else _f64(init_state).copy()
    _load().la_oracle_state(_p(k), _p(v), seg.ctypes.data_as(_I64), nseq, H, D, _p(st))
    return st


def backward(q, k, v, g, w, dout, cu_seqlens=None, eps=1e-6, init_state=None,
             d_final_state=None):
    """Gradient of the prefill (chain rule through Mechanism steps 4, 3, 2 in
    reverse).  dout: [T, H, D], the loss gradient w.r.t. the output;
    d_final_state: [nseq, H, D, D] or None, w.r.t. the final states.
    Returns dict(dq, dk, dv, dg [T, H, D], dw [H*D], d_init [nseq, H, D, D]) in float64.
    """
    q, k, v, g, w, dout = (_f64(a) for a in (q, k, v, g, w, dout))
    T, H, D = q.shape
    seg = _segments(T, cu_seqlens)
    nseq = len(seg) - 1
    init = _f64(init_state)
    dfin = _f64(d_final_state)
    for x, name in ((init, "init_state"), (dfin, "d_final_state")):
        if x is not None and x.shape != (nseq, H, D, D):
            raise ValueError(name + " shape")
    res = {n: np.empty((T, H, D), np.float64) for n in ("dq", "dk", "dv", "dg")}
    res["dw"] = np.empty(H * D, np.float64)
    res["d_init"] = np.empty((nseq, H, D, D), np.float64)
    _load().la_oracle_backward(_p(q), _p(k), _p(v), _p(g), _p(w), _p(dout),
                               seg.ctypes.data_as(_I64), nseq, H, D, float(eps), _p(init), _p(dfin),
                               _p(res["dq"]), _p(res["dk"]), _p(res["dv"]), _p(res["dg"]),
                               _p(res["dw"]), _p(res["d_init"]))
    return res


def layer(x, w_qkvg, w, w_out, head_dim=128, cu_seqlens=None, eps=1e-6, init_state=None,
          return_state=False):
    """The layer with its projections (Mechanism step 1: q, k, v and the gate are
    linear maps of the input; the output is mapped back to the hidden size):
    out = prefill(x Wq, x Wk, x Wv, x Wg) Wo, the matrix products in float64.
    x: [T, hidden]; w_qkvg: [4, hidden, H*D]; w: [H*D]; w_out: [H*D, hidden]."""
    x, w_qkvg, w_out = _f64(x), _f64(w_qkvg), _f64(w_out)
    T = x.shape[0]
    HD = w_qkvg.shape[2]
    D = int(head_dim)
    q, k, v, g = ((x @ w_qkvg[i]).reshape(T, HD // D, D) for i in range(4))
    res = prefill(q, k, v, g, w, cu_seqlens=cu_seqlens, eps=eps, init_state=init_state,
                  return_state=return_state)
    attn, fs = (res if return_state else (res, None))
    out = attn.reshape(T, HD) @ w_out
    return (out, fs) if return_state else out


ROPE_BASE = 1e7  # the model card: RoPE base frequency 10,000,000


def rope(x, cu_seqlens=None, rope_dim=None, base=ROPE_BASE):
    """Rotary embedding of x [T, H, D] at each token's position within its
    sequence, on the first rope_dim features (default D/2, half of the head
    dimension) in adjacent pairs."""
    x = _f64(x)
    T, H, D = x.shape
    seg = _segments(T, cu_seqlens)
    rd = D // 2 if rope_dim is None else int(rope_dim)
    if rd < 0 or rd > D or rd % 2:
        raise ValueError("rope_dim must be even and at most head_dim")
    y = np.empty_like(x)
    _load().la_oracle_rope(_p(x), _p(y), seg.ctypes.data_as(_I64), len(seg) - 1, H, D, rd,
                           float(base))
    return y


def softmax_attention(q, k, v, cu_seqlens=None, rope_dim=None, base=ROPE_BASE, scale=None,
                      rows=None):
    """The hybrid's softmax attention layer: causal softmax attention per
    sequence, q and k rotated at their positions (rope_dim default D/2, base
    10M), logits scaled by `scale` (default 1/sqrt(D)).  q, k, v: [T, H, D].
    rows: optional token indices to compute (the rest of the result is NaN)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, D = q.shape
    seg = _segments(T, cu_seqlens)
    rd = D // 2 if rope_dim is None else int(rope_dim)
    if rd < 0 or rd > D or rd % 2:
        raise ValueError("rope_dim must be even and at most head_dim")
    sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.full((T, H, D), np.nan)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if r is not None and (np.any(r < 0) or np.any(r >= T)):
        raise ValueError("rows out of range")
    rc = _load().la_oracle_softmax_attention(
        _p(q), _p(k), _p(v), seg.ctypes.data_as(_I64), len(seg) - 1, H, D, rd, float(base), sc,
        None if r is None else r.ctypes.data_as(_I64), 0 if r is None else len(r), _p(out))
    if rc != 0:
        raise MemoryError("oracle allocation failed")
    return out


def compare(out_dev, out_ref):
    """Error metrics measured after the epilogue, relative to max|out_ref|:
    (e_max, e_mean) = (max|d|, mean|d|) / max|out_ref| over the compared elements."""
    a = _f64(out_dev)
    b = _f64(out_ref)
    d = np.abs(a - b)
    m = float(np.max(np.abs(b))) if b.size else 0.0
    if m == 0.0:
        return float(d.max(initial=0.0)), float(d.mean() if d.size else 0.0)
    return float(d.max()) / m, float(d.mean()) / m
