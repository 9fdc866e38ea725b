"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each pin takes the oracle module (so the mutation test can run it against
copies of the oracle with a planted mistake) and raises AssertionError when
the oracle disagrees with:
  * a different algorithm (the quadratic left product, tests/brute.py);
  * closed forms derived by hand for special inputs;
  * invariants of the definition (causality, RMSNorm, head permutation,
    block-size invariance, decode-after-prefill, segment independence);
  * library routines for the elementwise functions (scipy.special.expit).
The layer is the Lightning Attention Mechanism of "Diving into MiniMax01 405B
MoE" (section "Hybrid Modeling"), under the causal reading with the current
token included.
"""
import math

import numpy as np
from scipy.special import expit

import brute

TIGHT = 1e-12


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    m = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / m)


def rnd(seed, shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def pin_elementwise(orc):
    """sigmoid/SiLU against scipy's expit and textbook identities."""
    xs = np.linspace(-30.0, 30.0, 241)
    for x in xs:
        s = orc.sigmoid(x)
        assert abs(s - expit(x)) <= 1e-15 + 1e-13 * abs(expit(x)), (x, s)
        assert abs(orc.silu(x) - x * expit(x)) <= 1e-13 * max(1.0, abs(x)), x
        assert abs(orc.sigmoid(x) + orc.sigmoid(-x) - 1.0) < 1e-15
        assert abs((orc.silu(x) - orc.silu(-x)) - x) < 1e-12 * max(1.0, abs(x))
    assert orc.sigmoid(0.0) == 0.5 and orc.silu(0.0) == 0.0
    # sigmoid(ln 3) = 3/4 exactly in real arithmetic
    assert abs(orc.sigmoid(math.log(3.0)) - 0.75) < 1e-15


def pin_brute_force(orc):
    """Recurrence == left product (Q~K~^T (.) M)V~ + Q~ S0 on tiny random inputs,
    several segment layouts (including empty segments) and initial states."""
    cases = [
        (1, 1, [0, 5]),
        (2, 3, [0, 7]),
        (3, 4, [0, 3, 3, 9, 10]),
        (2, 8, [0, 0, 16, 17, 40]),
    ]
    for ci, (H, D, seg) in enumerate(cases):
        T = seg[-1]
        q, k, v, g = (rnd(100 * ci + j, (T, H, D)) for j in range(4))
        w = rnd(100 * ci + 5, (H * D,), 0.3) + 1.0
        nseq = len(seg) - 1
        for init in (None, rnd(100 * ci + 6, (nseq, H, D, D), 0.5)):
            out, y = orc.prefill(q, k, v, g, w, cu_seqlens=seg, eps=1e-6, init_state=init,
                                 return_y=True)
            yb = brute.attention(q, k, v, seg, init)
            ob = brute.layer(q, k, v, g, w, seg, 1e-6, init)
            if T:
                assert rel(y, yb) < TIGHT, ("y", H, D, seg, rel(y, yb))
                assert rel(out, ob) < TIGHT, ("out", H, D, seg, rel(out, ob))


def pin_first_token(orc):
    """Closed form of the first token: y_0 = (q~_0 . k~_0) v~_0 + q~_0 S0."""
    H, D, T = 2, 6, 4
    q, k, v, g = (rnd(7 + j, (T, H, D)) for j in range(4))
    w = np.ones(H * D)
    s0 = rnd(11, (1, H, D, D))
    _, y = orc.prefill(q, k, v, g, w, init_state=s0, return_y=True)
    for h in range(H):
        qs, ks, vs = (a[0, h] * expit(a[0, h]) for a in (q, k, v))
        expect = np.dot(qs, ks) * vs + qs @ s0[0, h]
        assert rel(y[0, h], expect) < TIGHT


def pin_constant_closed_form(orc):
    """All-constant input, derived by hand: with q = k = v = c, s = SiLU(c),
    S0 = a * ones:  S_t = (a + (t+1) s^2) ones,  y_t = s D (a + (t+1) s^2) in
    every entry; every entry of a token is equal so mean(y^2) = y^2 and
    out_t = y_t / sqrt(y_t^2 + eps) * w * sigmoid(gam)."""
    H, D, T = 3, 5, 9
    for c, a, gam, wv, eps in ((1.0, 0.0, 0.0, 1.0, 1e-6), (-0.7, 0.25, 1.3, 0.5, 1e-2),
                               (0.02, 0.0, -2.0, 2.0, 1e-6)):
        s = c / (1.0 + math.exp(-c))
        q = np.full((T, H, D), c)
        g = np.full((T, H, D), gam)
        w = np.full(H * D, wv)
        init = np.full((1, H, D, D), a)
        out, y = orc.prefill(q, q, q, g, w, eps=eps, init_state=init, return_y=True)
        sg = 1.0 / (1.0 + math.exp(-gam))
        for t in range(T):
            yt = s * D * (a + (t + 1) * s * s)
            ot = yt / math.sqrt(yt * yt + eps) * wv * sg
            assert abs(y[t] - yt).max() <= 1e-12 * abs(yt) + 1e-300, (c, t)
            assert abs(out[t] - ot).max() <= 1e-12 * abs(ot) + 1e-300, (c, t)


def pin_rmsnorm_invariant(orc):
    """Per token: mean_{h,d} (out / (w sigmoid(g)))^2 = ms / (ms + eps) with
    ms = mean_{h,d} y^2 -- the norm runs over all heads of a token."""
    H, D, T = 4, 8, 12
    q, k, v, g = (rnd(20 + j, (T, H, D)) for j in range(4))
    w = rnd(25, (H * D,), 0.1) + 1.0
    for eps in (1e-6, 0.5):
        out, y = orc.prefill(q, k, v, g, w, eps=eps, return_y=True)
        z = out.reshape(T, -1) / (w[None, :] * expit(g.reshape(T, -1)))
        ms = np.mean(y.reshape(T, -1) ** 2, axis=1)
        lhs = np.mean(z * z, axis=1)
        assert rel(lhs, ms / (ms + eps)) < 1e-12
    # zero queries give y = 0 and an output of exactly 0 (eps avoids 0/0)
    out = orc.prefill(np.zeros((T, H, D)), k, v, g, w)
    assert np.all(out == 0.0)


def pin_causality(orc):
    """Changing token t's inputs leaves earlier outputs unchanged and changes
    token t itself (the diagonal is included); the norm couples heads."""
    H, D, T = 3, 4, 10
    q, k, v, g = (rnd(30 + j, (T, H, D)) for j in range(4))
    w = np.ones(H * D)
    base = orc.prefill(q, k, v, g, w)
    for t in (0, 4, 9):
        for arr_i in (1, 2):  # k and v of token t
            arrs = [q.copy(), k.copy(), v.copy()]
            arrs[arr_i][t] += 0.5
            o = orc.prefill(arrs[0], arrs[1], arrs[2], g, w)
            assert np.array_equal(o[:t], base[:t])
            assert rel(o[t], base[t]) > 1e-6
    # perturbing head 0 only changes head 1's output at that token (norm)
    q2 = q.copy()
    q2[5, 0] *= 3.0
    o = orc.prefill(q2, k, v, g, w)
    assert rel(o[5, 1], base[5, 1]) > 1e-9
    assert np.array_equal(o[:5], base[:5])


def pin_head_permutation(orc):
    """Permuting heads (q, k, v, g and the weight blocks) permutes the output."""
    H, D, T = 4, 3, 7
    q, k, v, g = (rnd(40 + j, (T, H, D)) for j in range(4))
    w = rnd(45, (H * D,), 0.2) + 1.0
    perm = np.array([2, 0, 3, 1])
    out = orc.prefill(q, k, v, g, w)
    wp = w.reshape(H, D)[perm].reshape(-1)
    outp = orc.prefill(q[:, perm], k[:, perm], v[:, perm], g[:, perm], wp)
    assert rel(outp, out[:, perm]) < TIGHT


def pin_blocked(orc):
    """Block-tiled form == token recurrence for block sizes 1, 7, 32, 64 and L;
    block 1 is the recurrence, block L the full masked product."""
    H, D = 2, 8
    seg = [0, 50, 50, 123]
    T = seg[-1]
    q, k, v, g = (rnd(50 + j, (T, H, D)) for j in range(4))
    w = rnd(55, (H * D,), 0.1) + 1.0
    init = rnd(56, (3, H, D, D), 0.3)
    ref, st = orc.prefill(q, k, v, g, w, cu_seqlens=seg, init_state=init, return_state=True)
    for blk in (1, 7, 32, 64, T):
        out, st2 = orc.prefill_blocked(q, k, v, g, w, blk, cu_seqlens=seg, init_state=init,
                                       return_state=True)
        assert rel(out, ref) < TIGHT, blk
        assert rel(st2, st) < TIGHT, blk


def pin_decode_after_prefill(orc):
    """Rows L..L+m-1 of a prefill of L+m tokens == a prefill of L tokens
    followed by m single-token decode steps carrying the state."""
    H, D, L, m = 3, 6, 11, 4
    q, k, v, g = (rnd(60 + j, (L + m, H, D)) for j in range(4))
    w = rnd(65, (H * D,), 0.1) + 1.0
    full = orc.prefill(q, k, v, g, w)
    _, st = orc.prefill(q[:L], k[:L], v[:L], g[:L], w, return_state=True)
    for i in range(m):
        t = L + i
        o, st = orc.decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], w, st)
        assert rel(o[0], full[t]) < TIGHT, i
    # state == S0 + K~^T V~ (matrix product from numpy)
    ks = k * expit(k)
    vs = v * expit(v)
    for h in range(H):
        assert rel(st[0, h], ks[:, h].T @ vs[:, h]) < TIGHT


def pin_segments_and_resume(orc):
    """Packed segments == separate calls; prefill(a+b) == prefill(b) resumed
    from the state after a; the state routine equals the prefill's state."""
    H, D = 2, 5
    lens = [6, 0, 13, 1]
    seg = np.concatenate([[0], np.cumsum(lens)])
    T = int(seg[-1])
    q, k, v, g = (rnd(70 + j, (T, H, D)) for j in range(4))
    w = np.ones(H * D)
    packed, st = orc.prefill(q, k, v, g, w, cu_seqlens=seg, return_state=True)
    for s in range(len(lens)):
        a, b = int(seg[s]), int(seg[s + 1])
        if a == b:
            assert np.all(st[s] == 0.0)
            continue
        o, st1 = orc.prefill(q[a:b], k[a:b], v[a:b], g[a:b], w, return_state=True)
        assert rel(packed[a:b], o) < TIGHT
        assert rel(st[s], st1[0]) < TIGHT
    assert rel(orc.state(k, v, cu_seqlens=seg), st) < TIGHT
    a = 9
    o_all, st_all = orc.prefill(q, k, v, g, w, return_state=True)
    _, st_a = orc.prefill(q[:a], k[:a], v[:a], g[:a], w, return_state=True)
    o_b, st_b = orc.prefill(q[a:], k[a:], v[a:], g[a:], w, init_state=st_a, return_state=True)
    assert rel(o_b, o_all[a:]) < TIGHT
    assert rel(st_b, st_all) < TIGHT


# ------------------------------------------------------------- backward
# The gradient of the layer (oracle.backward) is pinned to the derivative of
# the forward by central finite differences, to reverse-mode autodiff of an
# independent PyTorch statement of the forward, and to a closed form.

def _bwd_inputs(seed, T, H, D, nseq):
    q, k, v, g = (rnd(seed + i, (T, H, D)) for i in range(4))
    w = rnd(seed + 4, (H * D,), 0.5) + 1.0
    init = rnd(seed + 5, (nseq, H, D, D), 0.5)
    dout = rnd(seed + 6, (T, H, D))
    dfin = rnd(seed + 7, (nseq, H, D, D), 0.3)
    return q, k, v, g, w, init, dout, dfin


def pin_backward_finite_differences(orc):
    """Every gradient entry against a central difference of the oracle's own
    forward, loss = <out, dout> + <final state, dfin>; segments include an
    empty one."""
    T, H, D, seg, eps = 6, 2, 3, [0, 2, 2, 6], 1e-6
    q, k, v, g, w, init, dout, dfin = _bwd_inputs(71, T, H, D, 3)
    grads = orc.backward(q, k, v, g, w, dout, cu_seqlens=seg, eps=eps, init_state=init,
                         d_final_state=dfin)
    args = {"q": q, "k": k, "v": v, "g": g, "w": w, "init": init}

    def loss(a):
        out, fs = orc.prefill(a["q"], a["k"], a["v"], a["g"], a["w"], cu_seqlens=seg, eps=eps,
                              init_state=a["init"], return_state=True)
        return float(np.sum(out * dout) + np.sum(fs * dfin))

    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "w": "dw", "init": "d_init"}
    step = 1e-5
    for n, x in args.items():
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            a = {m: y.copy() for m, y in args.items()}
            a[n][idx] = x[idx] + step
            lp = loss(a)
            a[n][idx] = x[idx] - step
            lm = loss(a)
            fd[idx] = (lp - lm) / (2 * step)
        got = grads[names[n]]
        assert np.max(np.abs(got - fd)) <= 1e-6 * max(1.0, np.max(np.abs(fd))), (n, got, fd)


def _torch_forward(q, k, v, g, w, seg, eps, init):
    """Plain PyTorch statement of the layer (left product per segment and head)."""
    import torch
    silu = lambda x: x * torch.sigmoid(x)
    qs, ks, vs = silu(q), silu(k), silu(v)
    T, H, D = q.shape
    y = torch.zeros(T, H, D, dtype=q.dtype)
    finals = []
    for s in range(len(seg) - 1):
        a, b = seg[s], seg[s + 1]
        for h in range(H):
            Q, K, V = qs[a:b, h], ks[a:b, h], vs[a:b, h]
            y[a:b, h] = torch.tril(Q @ K.T) @ V + Q @ init[s, h]
            finals.append(init[s, h] + K.T @ V)
    fs = torch.stack(finals).reshape(len(seg) - 1, H, D, D)
    yf = y.reshape(T, H * D)
    r = torch.rsqrt(torch.mean(yf * yf, dim=1, keepdim=True) + eps)
    out = (yf * r * w * torch.sigmoid(g.reshape(T, H * D))).reshape(T, H, D)
    return out, fs


def pin_backward_autograd(orc):
    """All gradients against torch.autograd (float64, CPU) of the PyTorch forward."""
    import torch
    T, H, D, seg, eps = 29, 3, 5, [0, 11, 11, 29], 1e-6
    q, k, v, g, w, init, dout, dfin = _bwd_inputs(91, T, H, D, 3)
    grads = orc.backward(q, k, v, g, w, dout, cu_seqlens=seg, eps=eps, init_state=init,
                         d_final_state=dfin)
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, g, w, init)]
    out, fs = _torch_forward(*ts[:5], seg, eps, ts[5])
    L = (out * torch.tensor(dout)).sum() + (fs * torch.tensor(dfin)).sum()
    ref = torch.autograd.grad(L, ts)
    for n, r in zip(("dq", "dk", "dv", "dg", "dw", "d_init"), ref):
        assert rel(grads[n], r.numpy()) < 1e-11, (n, rel(grads[n], r.numpy()))


def pin_backward_final_state_only(orc):
    """dout = 0: only the final state carries gradient, so dq = dg = dw = 0,
    dL/dS0 = dfin, and every token sees dS_t = dfin: dk_t = (v~_t dfin^T) SiLU'(k_t),
    dv_t = (k~_t dfin) SiLU'(v_t), with SiLU' from scipy's expit."""
    T, H, D, seg = 9, 2, 4, [0, 4, 9]
    q, k, v, g, w, init, _, dfin = _bwd_inputs(113, T, H, D, 2)
    grads = orc.backward(q, k, v, g, w, np.zeros((T, H, D)), cu_seqlens=seg, init_state=init,
                         d_final_state=dfin)
    for n in ("dq", "dg", "dw"):
        assert np.all(grads[n] == 0.0), n
    assert rel(grads["d_init"], dfin) < TIGHT
    dsilu = lambda x: expit(x) * (1.0 + x * (1.0 - expit(x)))
    silu = lambda x: x * expit(x)
    for s in range(2):
        for t in range(seg[s], seg[s + 1]):
            for h in range(H):
                dk = (dfin[s, h] @ silu(v[t, h])) * dsilu(k[t, h])
                dv = (silu(k[t, h]) @ dfin[s, h]) * dsilu(v[t, h])
                assert rel(grads["dk"][t, h], dk) < TIGHT
                assert rel(grads["dv"][t, h], dv) < TIGHT


BACKWARD_PINS = [pin_backward_finite_differences, pin_backward_autograd,
                 pin_backward_final_state_only]


def pin_layer_composition(orc):
    """The layer with distinct scaled-identity projections (Wq = I, Wk = 2 I,
    Wv = -I, Wg = I / 2) and a permutation for Wo equals the prefill of
    (x, 2x, -x, x/2) with its outputs permuted: any mix-up of the four
    projections or of the output map changes the result."""
    T, H, D, seg = 12, 2, 3, [0, 5, 12]
    HD = H * D
    x = rnd(131, (T, HD))
    w = rnd(132, (HD,), 0.3) + 1.0
    eye = np.eye(HD)
    wq = np.stack([eye, 2 * eye, -eye, 0.5 * eye])
    perm = np.random.default_rng(133).permutation(HD)
    wo = eye[:, perm]
    got = orc.layer(x, wq, w, wo, head_dim=D, cu_seqlens=seg)
    xs = x.reshape(T, H, D)
    ref = orc.prefill(xs, 2 * xs, -xs, 0.5 * xs, w, cu_seqlens=seg).reshape(T, HD)[:, perm]
    assert rel(got, ref) < TIGHT

ALL_PINS = [pin_elementwise, pin_brute_force, pin_first_token, pin_constant_closed_form,
            pin_rmsnorm_invariant, pin_causality, pin_head_permutation, pin_blocked,
            pin_decode_after_prefill, pin_segments_and_resume] + BACKWARD_PINS + [pin_layer_composition]
# (the softmax pins are appended below, once defined)


# ------------------------------------------------------------ softmax layer
# The hybrid's softmax attention layer ("Diving into MiniMax01 405B MoE",
# section "Hybrid Modeling", 1/8 Softmax Attention; model card "2. Model
# Architecture", Positional Encoding): rotary embedding on half of the head
# dimension, base 10,000,000, causal softmax attention.

def _rope_complex(x, seg, rope_dim, base):
    """Rotary embedding written as complex multiplication (its form in the
    RoFormer paper): feature pairs (2i, 2i+1) read as z = x_2i + j x_2i+1,
    multiplied by exp(j pos base^(-2i/d)); a different formulation from the
    oracle's plane rotation."""
    y = np.array(x, np.float64, copy=True)
    pos = np.concatenate([np.arange(b - a) for a, b in zip(seg[:-1], seg[1:])]).astype(np.float64)
    z = y[..., 0:rope_dim:2] + 1j * y[..., 1:rope_dim:2]
    freq = np.exp(-np.log(base) * np.arange(0, rope_dim, 2) / rope_dim)
    z = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    y[..., 0:rope_dim:2] = z.real
    y[..., 1:rope_dim:2] = z.imag
    return y


def pin_rope(orc):
    """Rotary embedding: the page's base and fraction; equal to the complex
    form; position 0 and the unrotated half pass unchanged; each pair keeps its
    norm; <rope(q, m), rope(k, n)> depends only on m - n."""
    import json, os
    facts = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                        "page_facts.json")))
    assert orc.ROPE_BASE == facts["rope_base"]
    T, H, D = 13, 2, 16
    seg = np.array([0, 5, 5, 13])
    x = rnd(151, (T, H, D))
    y = orc.rope(x, cu_seqlens=seg)  # default: half of the head dimension
    assert rel(y, _rope_complex(x, seg, D // 2, facts["rope_base"])) < TIGHT
    assert np.array_equal(y[:, :, D // 2:], x[:, :, D // 2:])
    assert rel(y[[0, 5]], x[[0, 5]]) < TIGHT
    pn = lambda a: a[..., 0:D // 2:2] ** 2 + a[..., 1:D // 2:2] ** 2
    assert rel(pn(y), pn(x)) < TIGHT
    for rd, base in ((D, 10000.0), (4, 500.0)):
        assert rel(orc.rope(x, cu_seqlens=seg, rope_dim=rd, base=base),
                   _rope_complex(x, seg, rd, base)) < TIGHT
    # relative positions: the same q and k vectors at every position of one sequence
    L = 40
    qv, kv = rnd(152, (1, 1, D)), rnd(153, (1, 1, D))
    rq = orc.rope(np.repeat(qv, L, 0), rope_dim=D, base=50.0)[:, 0]
    rk = orc.rope(np.repeat(kv, L, 0), rope_dim=D, base=50.0)[:, 0]
    for m, n, c in ((7, 3, 11), (3, 7, 20), (0, 0, 39), (12, 30, 5)):
        assert abs(rq[m] @ rk[n] - rq[m + c] @ rk[n + c]) < 1e-10


def pin_softmax_closed_forms(orc):
    """The first token of every sequence returns its own value; with q = 0 all
    logits are equal, so token t returns the mean of v over its sequence's
    tokens up to and including t."""
    T, H, D = 17, 3, 8
    seg = np.array([0, 1, 9, 9, 17])
    q, k, v = rnd(161, (T, H, D)), rnd(162, (T, H, D)), rnd(163, (T, H, D))
    out = orc.softmax_attention(q, k, v, cu_seqlens=seg)
    for a in (0, 1, 9):
        assert rel(out[a], v[a]) < TIGHT
    out0 = orc.softmax_attention(np.zeros_like(q), k, v, cu_seqlens=seg)
    ref = np.empty_like(v)
    for a, b in zip(seg[:-1], seg[1:]):
        for t in range(a, b):
            ref[t] = v[a:t + 1].mean(axis=0)
    assert rel(out0, ref) < TIGHT


def pin_softmax_library(orc):
    """With the rotation switched off, each sequence equals torch's causal
    scaled_dot_product_attention in float64 (default scale 1/sqrt(D), and an
    explicit one)."""
    import torch
    T, H, D = 23, 2, 16
    seg = np.array([0, 10, 23])
    q, k, v = rnd(171, (T, H, D)), rnd(172, (T, H, D)), rnd(173, (T, H, D))
    for scale in (None, 0.37):
        out = orc.softmax_attention(q, k, v, cu_seqlens=seg, rope_dim=0, scale=scale)
        for a, b in zip(seg[:-1], seg[1:]):
            tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x[a:b].transpose(1, 0, 2)))
                          for x in (q, k, v))
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                                   scale=scale)
            assert rel(out[a:b], ref.numpy().transpose(1, 0, 2)) < 1e-12


def pin_softmax_rope_composition(orc):
    """Attention with the rotation equals attention without it on inputs
    rotated beforehand (complex form, positions restarting in every sequence);
    packing sequences together changes nothing; rows computed alone match."""
    T, H, D = 29, 2, 16
    seg = np.array([0, 11, 11, 29])
    q, k, v = rnd(181, (T, H, D), 2.0), rnd(182, (T, H, D), 2.0), rnd(183, (T, H, D))
    base = 30.0  # a small base, so that every pair turns noticeably over a few tokens
    out = orc.softmax_attention(q, k, v, cu_seqlens=seg, base=base)
    ref = orc.softmax_attention(_rope_complex(q, seg, D // 2, base),
                                _rope_complex(k, seg, D // 2, base), v, cu_seqlens=seg,
                                rope_dim=0)
    assert rel(out, ref) < 1e-12
    for a, b in zip(seg[:-1], seg[1:]):
        if b > a:
            alone = orc.softmax_attention(q[a:b], k[a:b], v[a:b], base=base)
            assert rel(out[a:b], alone) < TIGHT
    rows = [28, 0, 11, 17]
    part = orc.softmax_attention(q, k, v, cu_seqlens=seg, base=base, rows=rows)
    assert rel(part[rows], out[rows]) < TIGHT
    assert np.isnan(part[1]).all()


SOFTMAX_PINS = [pin_rope, pin_softmax_closed_forms, pin_softmax_library,
                pin_softmax_rope_composition]

ALL_PINS = ALL_PINS + SOFTMAX_PINS
