"""The softmax attention layer on the GPU against the oracle (needs an MI355X).

The hybrid's softmax layer: rotary embedding on half of the head dimension
(base 1e7 by default), causal softmax attention per sequence.  Outputs are
compared with oracle.softmax_attention on the same bf16 inputs, to the bf16 bar
(e_max relative to the largest reference magnitude).  Shapes span several
128-query tiles and 64-key blocks with ragged tails; varlen packs include
empty and one-token sequences; the full 8192-token x 64-head workload is
checked on sampled tokens (every head), which the oracle computes one by one.
The decode step against a KV cache is checked against the oracle's attention
row of the new token, against a prefill of the same tokens, and for its
handling of cache lengths out of range.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check, dev, host, say
import long_context_attn_amd as la
from long_context_attn_amd import synth

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def qkv(T, H, D, key, scale=1.0):
    """Seeded bf16 q, k, v [T, H, D] (the values the oracle sees are the bf16 ones)."""
    return [synth.normal((synth.SEED, 95, key, i), (T, H, D), scale=scale, bf16=True)
            for i in range(3)]


@pytest.mark.parametrize("B,N,H,rope_dim,base,scale", [
    (2, 300, 3, 64, 1e7, 1.0),      # the model's rotation; ragged last tile and block
    (1, 700, 2, 128, 100.0, 1.0),   # all features turned, a fast-turning base
    (2, 129, 2, 0, 1e7, 1.0),       # no rotation
    (1, 1000, 2, 64, 1e4, 3.0),     # peaked logits: the running maximum moves often
    (3, 1, 1, 64, 1e7, 1.0),        # one token per row
])
def test_softmax_batch(B, N, H, rope_dim, base, scale):
    D = 128
    T = B * N
    q, k, v = qkv(T, H, D, key=B * 1000 + N, scale=scale)
    seg = np.arange(B + 1) * N
    say("softmax B", B, "N", N, "H", H, "rope_dim", rope_dim, "base", base)
    ref = oracle.softmax_attention(q, k, v, cu_seqlens=seg, rope_dim=rope_dim, base=base)
    out = la.softmax_prefill(*(dev(a, BF).view(B, N, H, D) for a in (q, k, v)),
                             rope_dim=rope_dim, rope_base=base)
    torch.cuda.synchronize()
    check(host(out).reshape(T, H, D), ref, BF,
          "softmax B=%d N=%d H=%d rope_dim=%d base=%g" % (B, N, H, rope_dim, base))


def test_softmax_varlen():
    D, H = 128, 2
    lens = [0, 1, 127, 128, 129, 300, 0, 5, 700]
    seg = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(seg[-1])
    q, k, v = qkv(T, H, D, key=77)
    ref = oracle.softmax_attention(q, k, v, cu_seqlens=seg)
    cu = torch.from_numpy(seg.astype(np.int32)).cuda()
    say("softmax varlen", lens)
    out = la.softmax_prefill_varlen(*(dev(a, BF) for a in (q, k, v)), cu)
    torch.cuda.synchronize()
    check(out, ref, BF, "softmax varlen")
    # positions restart in every sequence: each equals its own call
    for a, b in zip(seg[:-1], seg[1:]):
        if b - a > 0:
            alone = la.softmax_prefill(*(dev(x[a:b], BF).view(1, b - a, H, D) for x in (q, k, v)))
            torch.cuda.synchronize()
            assert torch.equal(alone.view(b - a, H, D), out[a:b])


def test_softmax_empty_and_scale():
    H, D = 2, 128
    x = torch.empty(2, 0, H, D, device="cuda", dtype=BF)
    say("softmax with no tokens")
    assert la.softmax_prefill(x, x, x).numel() == 0
    T = 200
    q, k, v = qkv(T, H, D, key=5)
    say("softmax explicit scale")
    ref = oracle.softmax_attention(q, k, v, scale=0.02)
    out = la.softmax_prefill(*(dev(a, BF).view(1, T, H, D) for a in (q, k, v)), scale=0.02)
    torch.cuda.synchronize()
    check(host(out).reshape(T, H, D), ref, BF, "softmax scale 0.02")


def test_softmax_8k_workload_sampled():
    """The 8192-token x 64-head workload (bf16, rotation on 64 of 128 features,
    base 1e7), in the launch configuration the bench times; the oracle computes
    sampled tokens (all 64 heads each), including the first and last token and
    both sides of tile and block boundaries."""
    N, H, D = 8192, 64, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2025 * 1000 + 95)
    x = [torch.randn(1, N, H, D, device="cuda", generator=gen).to(BF) for _ in range(3)]
    say("softmax 8K: inputs ready")
    out = la.softmax_prefill(*x)
    torch.cuda.synchronize()
    say("softmax 8K: GPU done")
    rows = [0, 1, 63, 64, 127, 128, 129, 1000, 2047, 2048, 4095, 5555, 8063, 8064, 8190, 8191]
    q, k, v = (host(t).reshape(N, H, D) for t in x)
    ref = oracle.softmax_attention(q, k, v, rows=rows)
    check(host(out).reshape(N, H, D)[rows], ref[rows], BF, "softmax 8K x 64 heads, sampled")


def _decode_case(lens, H, max_len, key):
    """Raw q, k, v of L + 1 tokens per sequence.  The caches hold the first L
    keys rotated (by the oracle, rounded to bf16) and values, and stale values
    in slot L; the step's expected output is row L of the oracle's attention on
    the raw tokens, and slot L must end up holding the new key rotated at L."""
    D = 128
    S = len(lens)
    kc = np.zeros((S, max_len, H, D), np.float32)
    vc = np.zeros((S, max_len, H, D), np.float32)
    qn, kn, vn = (np.zeros((S, H, D), np.float32) for _ in range(3))
    ref = np.zeros((S, H, D))
    new_k, new_v = [], []
    for s_, L in enumerate(lens):
        q, k, v = qkv(L + 1, H, D, key=key + s_)
        kr = host(dev(oracle.rope(k), BF))  # the cache's keys: rotated, bf16
        kc[s_, :L] = kr[:L]
        vc[s_, :L] = v[:L]
        kc[s_, L] = -7.0  # stale contents of the slot the step writes
        vc[s_, L] = 3.0
        qn[s_], kn[s_], vn[s_] = q[L], k[L], v[L]
        ref[s_] = oracle.softmax_attention(q, k, v, rows=[L])[L]
        new_k.append(kr[L])
        new_v.append(v[L])
    # head-major caches [S, H, max_len, D]
    kc, vc = (np.ascontiguousarray(c.transpose(0, 2, 1, 3)) for c in (kc, vc))
    return qn, kn, vn, kc, vc, ref, new_k, new_v


@pytest.mark.parametrize("lens,H,max_len", [
    ([0, 1, 511, 512, 513, 1500, 7], 2, 1600),   # empty cache, one key, split edges
    ([767, 768, 769, 1535, 1536, 3], 2, 2400),    # edges of the 768-key ranges
    ([4000, 2048], 4, 4096),
])
def test_softmax_decode(lens, H, max_len):
    qn, kn, vn, kc, vc, ref, new_k, new_v = _decode_case(lens, H, max_len, 300 + len(lens))
    say("softmax decode lens", lens, "H", H, "max_len", max_len)
    kcd, vcd = dev(kc, BF), dev(vc, BF)
    ln = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = la.softmax_decode(dev(qn, BF), dev(kn, BF), dev(vn, BF), kcd, vcd, ln)
    torch.cuda.synchronize()
    check(out, ref, BF, "softmax decode lens=%s" % lens)
    # the new key (rotated at its position) and value were appended at slot L
    for s_, L in enumerate(lens):
        np.testing.assert_allclose(host(kcd[s_, :, L]), new_k[s_], rtol=0,
                                   atol=2e-2 * np.abs(new_k[s_]).max())
        assert np.array_equal(host(vcd[s_, :, L]), new_v[s_])
    assert torch.equal(ln, torch.tensor(lens, dtype=torch.int32, device="cuda"))  # not advanced


def test_softmax_decode_steps_match_prefill():
    """Prefill-free generation: starting from an empty cache, N decode steps
    (the caller advancing the lengths) give the same outputs as one causal
    prefill of the N tokens."""
    H, D, N = 2, 128, 300
    q, k, v = qkv(N, H, D, key=401)
    kc = torch.zeros(1, H, N, D, device="cuda", dtype=BF)
    vc = torch.zeros_like(kc)
    ln = torch.zeros(1, dtype=torch.int32, device="cuda")
    qd, kd, vd = (dev(x, BF) for x in (q, k, v))
    say("softmax decode: 300 steps from an empty cache")
    outs = []
    for t in range(N):
        outs.append(la.softmax_decode(qd[t:t + 1], kd[t:t + 1], vd[t:t + 1], kc, vc, ln))
        ln += 1
    torch.cuda.synchronize()
    dec = torch.cat(outs)
    pre = la.softmax_prefill(*(x.view(1, N, H, D) for x in (qd, kd, vd))).view(N, H, D)
    ref = oracle.softmax_attention(q, k, v)
    check(dec, ref, BF, "softmax decode steps vs oracle")
    check(dec, host(pre).astype(np.float64), BF, "softmax decode steps vs the GPU prefill")


def test_softmax_decode_bad_length_is_reported():
    H, D, max_len = 2, 128, 64
    q, k, v = qkv(3, H, D, key=402)
    kc = torch.zeros(3, H, max_len, D, device="cuda", dtype=BF)
    vc = torch.zeros_like(kc)
    ln = torch.tensor([5, max_len, -1], dtype=torch.int32, device="cuda")
    out = torch.full((3, H, D), 9.0, device="cuda", dtype=BF)
    ws = torch.empty(la.softmax_decode_workspace_size(3, max_len, H, D), dtype=torch.uint8,
                     device="cuda")
    say("softmax decode with out-of-range lengths")
    la.softmax_decode(*(dev(x, BF) for x in (q, k, v)), kc, vc, ln, out=out, workspace=ws)
    torch.cuda.synchronize()
    status = ws[:12].view(torch.int32).cpu().tolist()
    assert status == [0, 1, 1]
    assert torch.all(out[1:] == 9.0)           # skipped sequences keep their output
    assert torch.count_nonzero(kc[1:]) == 0    # and their caches


@pytest.mark.slow
def test_softmax_decode_bench_shape():
    """One decode step at the shape bench.py times: 32 sequences x 64 heads,
    caches of max_len 16384 holding 1024..16383 keys (lengths from a seeded
    stream).  Six seeded sequences and the longest one carry seeded tokens and
    are compared with the oracle's attention row of the new token (every
    head); the others hold plausible filler and only have to run."""
    S, H, D, max_len = 32, 64, 128, 16384
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([synth.SEED, 96, 5, 0])))
    lens = [int(x) for x in g.integers(1024, max_len, size=S)]
    picks = sorted(set(synth.pick(6, S, 96, 1)) | {int(np.argmax(lens))})
    say("softmax decode bench shape: lengths", lens, "compared", picks)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2025 * 1000 + 97)
    kc = torch.empty(S, H, max_len, D, device="cuda", dtype=BF)
    vc = torch.empty_like(kc)
    for t in (kc, vc):
        for i in range(S):
            t[i].normal_(generator=gen)
    qn = torch.randn(S, H, D, device="cuda", generator=gen).to(BF)
    kn, vn = torch.randn_like(qn), torch.randn_like(qn)
    refs = {}
    for s_ in picks:
        L = lens[s_]
        q, k, v = qkv(L + 1, H, D, key=500 + s_)
        kr = host(dev(oracle.rope(k[:L]), BF))  # the cache's keys: rotated, bf16
        kc[s_, :, :L] = dev(np.ascontiguousarray(kr.transpose(1, 0, 2)), BF)
        vc[s_, :, :L] = dev(np.ascontiguousarray(v[:L].transpose(1, 0, 2)), BF)
        qn[s_], kn[s_], vn[s_] = dev(q[L], BF), dev(k[L], BF), dev(v[L], BF)
        refs[s_] = oracle.softmax_attention(q, k, v, rows=[L])[L]
    ln = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ws = torch.empty(la.softmax_decode_workspace_size(S, max_len, H, D), dtype=torch.uint8,
                     device="cuda")
    out = la.softmax_decode(qn, kn, vn, kc, vc, ln, workspace=ws)
    torch.cuda.synchronize()
    assert ws[:4 * S].view(torch.int32).cpu().tolist() == [0] * S
    o = host(out)
    check(o[picks], np.stack([refs[s_] for s_ in picks]), BF,
          "softmax decode 32 x 64 heads, caches 1K-16K, sequences %s" % picks)
