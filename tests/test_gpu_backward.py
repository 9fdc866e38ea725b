"""Backward pass on the GPU against the oracle's gradient (needs an MI355X).

Every gradient (dq, dk, dv, dgate, dweight, and the gradient w.r.t. the
initial states) is compared with oracle.backward on the same seeded inputs,
with a gradient reaching the final states as well as the output.  Metric:
the layer's e_max / e_mean, relative to the largest reference magnitude of
each tensor, against the bar of the input dtype.  fp32 inputs take the
portable fp32 kernels (every tensor within 1e-4).  bf16 inputs at head_dim
128 take the MFMA walks, whose operands (SiLU outputs, dy, the running
state) are bf16 as in the forward: every gradient, including the fp32
dweight and initial-state gradient, is then held to the bf16 bar.

The backward from saved activations (a prefill that keeps y and the chunk
states) is held to the same bar against the oracle, and compared with the
recomputing backward, which it matches bit for bit on these shapes.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check, dev, host, inputs, say
import long_context_attn_amd as la
from long_context_attn_amd import synth

pytestmark = pytest.mark.gpu

def rnd(seed, shape, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def compare(grads, ref, dtype, what):
    dq, dk, dv, dg, dw, d_init = grads
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv), ("dg", dg)):
        check(host(got).reshape(ref[name].shape), ref[name], dtype, "%s %s" % (what, name))
    for name, got in (("dw", dw), ("d_init", d_init)):
        if got is not None:
            check(host(got), ref[name], dtype, "%s %s" % (what, name))


def batch_case(B, N, H, D, dtype, dist, key, with_states=True):
    T = B * N
    q, k, v, g, w = inputs(T, H, D, dist, bf16=dtype == torch.bfloat16, key=key)
    dout = rnd(key + 100, (T, H, D))
    if dtype == torch.bfloat16:
        dout = host(dev(dout, torch.bfloat16))
    init = rnd(key + 101, (B, H, D, D), 0.5) if with_states else None
    dfin = rnd(key + 102, (B, H, D, D), 0.1) if with_states else None
    seg = np.arange(B + 1) * N
    ref = oracle.backward(q, k, v, g, w, dout, cu_seqlens=seg, init_state=init, d_final_state=dfin)
    return (q, k, v, g, w, dout, init, dfin), ref


def run_batch(args, B, N, H, D, dtype, block, chunk):
    q, k, v, g, w, dout, init, dfin = args
    x = [dev(a, dtype).view(B, N, H, D) for a in (q, k, v, g)]
    gd = dev(dout, dtype).view(B, N, H, D)
    st = lambda a: None if a is None else torch.from_numpy(a).cuda()
    grads = la.backward(*x, dev(w, dtype), gd, block=block, initial_state=st(init),
                        d_final_state=st(dfin), return_d_initial_state=True, chunk_tokens=chunk)
    torch.cuda.synchronize()
    dq, dk, dv, dg, dw, d_init = grads
    T = B * N
    return tuple(t.view(T, H, D) for t in (dq, dk, dv, dg)) + (dw, d_init)


@pytest.mark.parametrize("D,block", [(16, 16), (32, 32), (64, 64), (128, 32), (128, 64)])
def test_backward_fp32_shapes(D, block):
    B, N, H = 2, 301, 3
    args, ref = batch_case(B, N, H, D, torch.float32, "unit", 21)
    for chunk in (0, block, 4 * block):
        say("backward fp32 D", D, "block", block, "chunk", chunk)
        grads = run_batch(args, B, N, H, D, torch.float32, block, chunk)
        compare(grads, ref, torch.float32, "fp32 D=%d chunk=%d" % (D, chunk))


@pytest.mark.parametrize("D,block,dist", [(128, 64, "minimax"), (128, 64, "unit"), (64, 32, "unit")])
def test_backward_bf16(D, block, dist):
    B, N, H = 2, 700, 4
    args, ref = batch_case(B, N, H, D, torch.bfloat16, dist, 22)
    for chunk in (0, 2 * block):
        say("backward bf16 D", D, dist, "chunk", chunk)
        grads = run_batch(args, B, N, H, D, torch.bfloat16, block, chunk)
        compare(grads, ref, torch.bfloat16, "bf16 D=%d %s chunk=%d" % (D, dist, chunk))


def test_backward_bf16_without_initial_gradient():
    """No gradient w.r.t. the initial states requested: the MFMA path then
    skips each sequence's first chunk sum of q~^T dy (it only feeds that
    gradient); every other gradient must be unchanged."""
    B, N, H, D = 2, 700, 4, 128
    args, ref = batch_case(B, N, H, D, torch.bfloat16, "unit", 25)
    q, k, v, g, w, dout, init, dfin = args
    x = [dev(a, torch.bfloat16).view(B, N, H, D) for a in (q, k, v, g)]
    gd = dev(dout, torch.bfloat16).view(B, N, H, D)
    for chunk in (0, 128):
        say("backward bf16 without d_initial_state, chunk", chunk)
        dq, dk, dv, dg, dw, d_init = la.backward(
            *x, dev(w, torch.bfloat16), gd, block=64, initial_state=torch.from_numpy(init).cuda(),
            d_final_state=torch.from_numpy(dfin).cuda(), chunk_tokens=chunk)
        torch.cuda.synchronize()
        assert d_init is None
        T = B * N
        compare(tuple(t.view(T, H, D) for t in (dq, dk, dv, dg)) + (dw, None), ref,
                torch.bfloat16, "bf16 no d_init chunk=%d" % chunk)


def test_backward_long_norm_groups():
    """More than 2048 x 8 tokens: the norm backward's workgroups take 11 tokens
    each (1910 of them, the last with one token), so each dweight partial row
    sums 11 tokens."""
    B, N, H, D = 1, 21000, 2, 128
    args, ref = batch_case(B, N, H, D, torch.bfloat16, "unit", 24)
    say("backward bf16 21000 tokens x 2 heads")
    grads = run_batch(args, B, N, H, D, torch.bfloat16, 64, 0)
    compare(grads, ref, torch.bfloat16, "bf16 21000 tokens")


def test_backward_without_states():
    B, N, H, D = 1, 200, 2, 64
    args, ref = batch_case(B, N, H, D, torch.float32, "unit", 23, with_states=False)
    say("backward without initial / final states")
    q, k, v, g, w, dout, _, _ = args
    x = [dev(a, torch.float32).view(B, N, H, D) for a in (q, k, v, g, dout)]
    dq, dk, dv, dg, dw, d_init = la.backward(*x[:4], dev(w, torch.float32), x[4], block=32)
    torch.cuda.synchronize()
    assert d_init is None
    compare((dq.view(N, H, D), dk.view(N, H, D), dv.view(N, H, D), dg.view(N, H, D), dw, None),
            ref, torch.float32, "no states")


@pytest.mark.parametrize("dtype,D,block", [(torch.float32, 64, 32), (torch.bfloat16, 128, 64)])
def test_backward_varlen(dtype, D, block):
    lens = [0, 1, 63, 64, 65, 300, 0, 3, 2 * block + 7]
    seg = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, H, nseq = int(seg[-1]), 3, len(lens)
    q, k, v, g, w = inputs(T, H, D, "unit", bf16=dtype == torch.bfloat16, key=24)
    dout = rnd(124, (T, H, D))
    if dtype == torch.bfloat16:
        dout = host(dev(dout, torch.bfloat16))
    init = rnd(125, (nseq, H, D, D), 0.5)
    dfin = rnd(126, (nseq, H, D, D), 0.1)
    ref = oracle.backward(q, k, v, g, w, dout, cu_seqlens=seg, init_state=init, d_final_state=dfin)
    cu = torch.from_numpy(seg.astype(np.int32)).cuda()
    for chunk in (0, block):
        say("backward varlen", dtype, "chunk", chunk)
        grads = la.backward_varlen(*(dev(a, dtype) for a in (q, k, v, g, w, dout)), cu,
                                   block=block, initial_state=torch.from_numpy(init).cuda(),
                                   d_final_state=torch.from_numpy(dfin).cuda(),
                                   return_d_initial_state=True, chunk_tokens=chunk)
        torch.cuda.synchronize()
        compare(grads, ref, dtype, "varlen chunk=%d" % chunk)
        # an empty sequence passes the final-state gradient through unchanged
        d_init = host(grads[5])
        for s, L in enumerate(lens):
            if L == 0:
                assert np.array_equal(d_init[s], dfin[s])
        # without the initial-state gradient (each sequence's first chunk sum
        # of q~^T dy is then skipped) every other gradient is bit-identical
        again = la.backward_varlen(*(dev(a, dtype) for a in (q, k, v, g, w, dout)), cu,
                                   block=block, initial_state=torch.from_numpy(init).cuda(),
                                   d_final_state=torch.from_numpy(dfin).cuda(), chunk_tokens=chunk)
        torch.cuda.synchronize()
        assert again[5] is None
        for a, b in zip(again[:5], grads[:5]):
            assert torch.equal(a, b)


def test_backward_empty():
    H, D = 2, 32
    x = torch.empty(3, 0, H, D, device="cuda")
    w = torch.randn(H * D, device="cuda")
    dfin = torch.randn(3, H, D, D, device="cuda")
    say("backward with no tokens")
    dq, dk, dv, dg, dw, d_init = la.backward(x, x, x, x, w, x, block=32, d_final_state=dfin,
                                             return_d_initial_state=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw) == 0
    assert torch.equal(d_init, dfin)


@pytest.mark.slow
def test_backward_8k_workload():
    """The full 8192-token x 64-head bf16 workload, every gradient against the oracle."""
    N, H, D = 8192, 64, 128
    q, k, v, g, w = synth.layer_inputs(synth.PREFILL_8K, N, H, D, "minimax", threads=16)
    dout = host(dev(rnd(8192, (N, H, D)), torch.bfloat16))
    say("backward 8K: inputs ready")
    x = [dev(a, torch.bfloat16).view(1, N, H, D) for a in (q, k, v, g, dout)]
    wd = dev(w, torch.bfloat16)
    grads = la.backward(*x[:4], wd, x[4], return_d_initial_state=True)
    torch.cuda.synchronize()
    say("backward 8K: GPU done")
    # the training order at the same shape: a saving prefill, then the
    # backward from its activations
    _, saved = la.prefill(*x[:4], wd, save_for_backward=True, check=True)
    from_saved = la.backward(*x[:4], wd, x[4], return_d_initial_state=True, saved=saved,
                             check=True)
    torch.cuda.synchronize()
    grads_close(grads, from_saved, "backward 8K")
    del saved, from_saved
    ref = oracle.backward(q, k, v, g, w, dout)
    dq, dk, dv, dg, dw, d_init = grads
    compare(tuple(t.view(N, H, D) for t in (dq, dk, dv, dg)) + (dw, d_init), ref, torch.bfloat16,
            "backward 8K x 64 heads")


def grads_close(a, b, what, bar=1e-2):
    """Two GPU gradient sets that differ only where y was rounded once more:
    every tensor within `bar` of the largest magnitude of the first."""
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dw", "d_init"), a, b):
        if x is None:
            assert y is None
            continue
        scale = max(x.float().abs().max().item(), 1e-30)
        err = (x.float() - y.float()).abs().max().item() / scale
        say("%s %s: saved vs recomputed, max rel diff %.2e" % (what, name, err))
        assert err < bar


@pytest.mark.parametrize("B,N,H", [(2, 1000, 3), (1, 777, 2)])
def test_backward_from_saved_activations(B, N, H):
    """A prefill that saves y and the chunk states gives the same outputs as the
    plain prefill (bit for bit); the backward from them matches the oracle, and
    the backward that recomputes them to bf16 rounding."""
    D, dtype = 128, torch.bfloat16
    args, ref = batch_case(B, N, H, D, dtype, "unit", key=61)
    q, k, v, g, w, dout, init, dfin = args
    x = [dev(a, dtype).view(B, N, H, D) for a in (q, k, v, g)]
    wd = dev(w, dtype)
    gd = dev(dout, dtype).view(B, N, H, D)
    st = lambda a: torch.from_numpy(a).cuda()
    say("prefill with saved activations B", B, "N", N, "H", H)
    plain, fs_plain = la.prefill(*x, wd, initial_state=st(init), return_final_state=True)
    out, fs, saved = la.prefill(*x, wd, initial_state=st(init), return_final_state=True,
                                save_for_backward=True, check=True)
    torch.cuda.synchronize()
    assert saved.numel() == la.saved_size(B * N, B, H, D)
    assert torch.equal(out, plain) and torch.equal(fs, fs_plain)
    # y as saved: the oracle's pre-norm output, to the bf16 bar
    y_saved = saved[:B * N * H * D * 2].view(torch.bfloat16).view(B * N, H, D)
    _, y_ref = oracle.prefill(q, k, v, g, w, cu_seqlens=np.arange(B + 1) * N, init_state=init,
                              return_y=True)
    check(host(y_saved), y_ref, dtype, "saved y")
    say("backward from the saved activations")
    kw = dict(initial_state=st(init), d_final_state=st(dfin), return_d_initial_state=True)
    from_saved = la.backward(*x, wd, gd, saved=saved, check=True, **kw)
    recomputed = la.backward(*x, wd, gd, **kw)
    torch.cuda.synchronize()
    T = B * N
    flat = lambda gr: tuple(t.view(T, H, D) for t in gr[:4]) + tuple(gr[4:])
    compare(flat(from_saved), ref, dtype, "from saved")
    grads_close(flat(recomputed), flat(from_saved), "B=%d N=%d" % (B, N))


def test_backward_varlen_from_saved_activations():
    """Packed sequences (empty ones, several chunks each at 64-token chunks)."""
    D, dtype, H = 128, torch.bfloat16, 3
    lens = [0, 1, 200, 64, 0, 331]
    seg = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, nseq = int(seg[-1]), len(lens)
    q, k, v, g, w = inputs(T, H, D, "unit", key=62)
    dout = host(dev(rnd(162, (T, H, D)), dtype))
    init = rnd(163, (nseq, H, D, D), 0.5)
    dfin = rnd(164, (nseq, H, D, D), 0.1)
    ref = oracle.backward(q, k, v, g, w, dout, cu_seqlens=seg, init_state=init, d_final_state=dfin)
    cu = torch.from_numpy(seg.astype(np.int32)).cuda()
    x = [dev(a, dtype) for a in (q, k, v, g, w)]
    st = lambda a: torch.from_numpy(a).cuda()
    for chunk in (0, 64):
        say("varlen saved activations, chunk", chunk)
        plain = la.prefill_varlen(*x, cu, initial_state=st(init), chunk_tokens=chunk)
        out, saved = la.prefill_varlen(*x, cu, initial_state=st(init), chunk_tokens=chunk,
                                       save_for_backward=True, check=True)
        torch.cuda.synchronize()
        assert torch.equal(out, plain)
        kw = dict(initial_state=st(init), d_final_state=st(dfin), return_d_initial_state=True,
                  chunk_tokens=chunk)
        from_saved = la.backward_varlen(*x, dev(dout, dtype), cu, saved=saved, check=True, **kw)
        recomputed = la.backward_varlen(*x, dev(dout, dtype), cu, **kw)
        torch.cuda.synchronize()
        compare(from_saved, ref, dtype, "varlen from saved chunk=%d" % chunk)
        grads_close(recomputed, from_saved, "varlen chunk=%d" % chunk)
