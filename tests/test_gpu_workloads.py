"""Full-size workloads on the GPU against the CPU oracle (needs an MI355X).

Every test runs the library at the workload's real shape and in the launch
configuration bench.py times (the library's automatic chunk length), then
compares what the fp64 oracle can compute in seconds:

  * prefill, 8192 tokens x 64 heads: every output and the final state, for the
    automatic configuration (2048-token chunks) and for 1024-token chunks;
    the state-only pass's final state;
  * decode, 256 sequences x 64 heads, 64 steps: each step's outputs and the
    final states of four seeded sequences whose initial states the oracle
    built from their seeded prefixes;
  * varlen, 1,048,576 packed tokens (automatic chunks of 8192 tokens): every
    output and final state of three seeded sequences of at most 8192 tokens,
    packed among the others (also with 2048-token chunks); every output and
    final state, on all heads, of a seeded sequence of 16K-40K tokens (several
    chunks: the scanned states entering them); the longest sequence (about
    124K tokens, 16 chunks): its final state on four seeded heads and its
    last 1024 outputs, which the oracle computes from the GPU's state after
    the tokens before them (checked on the four heads on its own);
  * the layer with its projections at the shape bench.py times (8192
    tokens, hidden 6144, 64 heads): every output;
  * one sequence of 1,048,576 tokens: the first 2048 outputs; the state after
    1,047,552 tokens on four seeded heads; the last 1024 outputs, which the
    oracle computes from the GPU's state after 1,047,552 tokens (the four
    seeded heads of that state having been checked on their own).

Inputs the comparison does not see only have to be plausible and come from
the GPU's random generator; the compared parts come from the seeded streams.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from gpu_util import check, dev, host, rel_state, say
import long_context_attn_amd as la
from long_context_attn_amd import synth

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
H, D = 64, 128
# final-state bound for bf16 inputs (see test_gpu_parity.py): the MFMA path
# multiplies bf16-rounded SiLU(k) and SiLU(v), so the state is within 2^-8
STATE_TOL = 4e-3
THREADS = 16


def gpu_normal(shape, seed, scale=1.0):
    """Plausible bf16 N(0, scale^2) filler, drawn on the device in slices."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    t = torch.empty(shape, dtype=BF16, device="cuda")
    flat = t.view(shape[0], -1)
    step = max(1, (1 << 28) // flat.shape[1])
    for a in range(0, shape[0], step):
        b = min(shape[0], a + step)
        x = torch.randn(b - a, flat.shape[1], device="cuda", generator=gen)
        flat[a:b] = (x * scale).to(BF16)
        del x
    return t


def put(dst, rows, heads, x):
    """dst[rows, heads, :] = x for a [T, H, D] device tensor and a host block."""
    xt = torch.from_numpy(x).to(BF16)
    if list(heads) == list(range(dst.shape[1])):
        dst[rows].copy_(xt)
    else:
        for i, h in enumerate(heads):
            dst[rows, h].copy_(xt[:, i])


def test_prefill_8k_workload():
    """The automatic configuration bench.py times, and 1024-token chunks (eight
    per sequence, 512 work items for 256 compute units), both against the
    oracle."""
    N = 8192
    q, k, v, g, w = synth.layer_inputs(synth.PREFILL_8K, N, H, D, "minimax", threads=THREADS)
    say("prefill 8K: inputs ready")
    args = [dev(a, BF16).view(1, N, H, D) for a in (q, k, v, g)] + [dev(w, BF16)]
    runs = {}
    for chunk in (0, 1024):
        say("prefill 8K: chunk_tokens", chunk)
        runs[chunk] = la.prefill(*args, return_final_state=True, chunk_tokens=chunk, check=True)
        torch.cuda.synchronize()
    # a second call of the benched configuration gives the same bits (the
    # cross-head sums are added in a fixed order; the store path keeps every
    # stored register allocated until the next barrier)
    say("prefill 8K: second call, bitwise")
    again = la.prefill(*args, return_final_state=True, check=True)
    torch.cuda.synchronize()
    assert torch.equal(again[0], runs[0][0]) and torch.equal(again[1], runs[0][1])
    del again
    say("prefill 8K: state-only pass")
    fs_only = la.state(args[1], args[2])
    torch.cuda.synchronize()
    ref, st = oracle.prefill(q, k, v, g, w, return_state=True)
    for chunk, (out, fs) in runs.items():
        check(host(out).reshape(N, H, D), ref, BF16, "prefill 8K x 64 heads, chunk_tokens %d" % chunk)
        err = rel_state(host(fs), st)
        say("prefill 8K chunk_tokens %d final state rel err %.2e" % (chunk, err))
        assert err < STATE_TOL
    err = rel_state(host(fs_only), st)
    say("state-only 8K x 64 heads: final state rel err %.2e" % err)
    assert err < STATE_TOL


@pytest.mark.slow
def test_decode_256_workload():
    S, steps = 256, 64
    lens = synth.decode_prefix_lengths(S)
    picks = synth.pick(4, S, synth.DECODE, 1)
    say("decode: sampled sequences", picks, "prefix lengths", [lens[s] for s in picks])
    # the other sequences' states only need a plausible magnitude
    state = gpu_normal((S, H, D, D), 31, 100.0).float()
    with ThreadPoolExecutor(len(picks)) as ex:
        kv = list(ex.map(lambda s: synth.decode_prefix_kv(s, lens[s], H, D), picks))
    ref_state = []
    for s, (k, v) in zip(picks, kv):
        s0 = oracle.state(k, v)[0].astype(np.float32)  # fp64 sum, rounded once to fp32
        state[s].copy_(torch.from_numpy(s0))
        ref_state.append(s0.astype(np.float64))
    del kv
    ref_state = np.stack(ref_state)
    say("decode: initial states ready")
    w = torch.ones(H * D, dtype=BF16, device="cuda")
    wh = np.ones(H * D, np.float32)
    out = torch.empty(S, H, D, dtype=BF16, device="cuda")
    worst = 0.0
    for step in range(steps):
        qs, ks, vs, gs = synth.decode_step_inputs(step, S, H, D)
        la.decode(*(dev(a, BF16) for a in (qs, ks, vs, gs)), w, state, out=out)
        torch.cuda.synchronize()
        ref, ref_state = oracle.decode(qs[picks], ks[picks], vs[picks], gs[picks], wh, ref_state)
        emax, _ = check(host(out)[picks], ref, BF16, "decode step %d" % step)
        worst = max(worst, emax)
    err = rel_state(host(state[picks]), ref_state)
    say("decode: worst step e_max %.2e, final states rel err %.2e" % (worst, err))
    assert err < 1e-4


@pytest.mark.slow
def test_varlen_1m_workload():
    T = 1 << 20
    lens = synth.varlen_lengths(T)
    cu = synth.cu_seqlens(lens)
    assert la.prefill_workspace_size(T, len(lens), H, D) == la.prefill_workspace_size(
        T, len(lens), H, D, 64, 8192)  # the automatic chunk at this size: 8192 tokens
    cand = [i for i, L in enumerate(lens) if 0 < L <= 8192 and i > 0]
    picks = [cand[i] for i in synth.pick(3, len(cand), synth.VARLEN_1M, 1)]
    # a sequence of several chunks, compared whole on every head
    mids = [i for i, L in enumerate(lens) if 16384 < L <= 40000]
    mid = mids[synth.pick(1, len(mids), synth.VARLEN_1M, 2)[0]]
    # the longest one: final state on four heads, last 1024 outputs
    far = int(np.argmax(lens))
    fheads = synth.pick_heads(4, H, synth.VARLEN_1M)
    say("varlen: %d sequences, sampled" % len(lens), [(s, lens[s]) for s in picks],
        "whole", (mid, lens[mid]), "longest", (far, lens[far]), "heads", fheads)
    q, k, v, g = (gpu_normal((T, H, D), 41 + t) for t in range(4))
    ids = (synth.Q, synth.K, synth.V, synth.G)
    wins = {}
    for s in picks + [mid]:
        a, b = int(cu[s]), int(cu[s + 1])
        ins = [synth.block_tensor(synth.VARLEN_1M, t, a, b, range(H), D, 1.0, threads=THREADS)
               for t in ids]
        for dst, x in zip((q, k, v, g), ins):
            put(dst, slice(a, b), range(H), x)
        wins[s] = ins
    fa, fb = int(cu[far]), int(cu[far + 1])
    fw = fb - 1024
    kf = synth.block_tensor(synth.VARLEN_1M, synth.K, fa, fb, fheads, D, 1.0, threads=THREADS)
    vf = synth.block_tensor(synth.VARLEN_1M, synth.V, fa, fb, fheads, D, 1.0, threads=THREADS)
    put(k, slice(fa, fb), fheads, kf)
    put(v, slice(fa, fb), fheads, vf)
    last = [synth.block_tensor(synth.VARLEN_1M, t, fw, fb, range(H), D, 1.0, threads=THREADS)
            for t in ids]
    for dst, x in zip((q, k, v, g), last):
        put(dst, slice(fw, fb), range(H), x)
    # the longest sequence's inputs on the four heads as the GPU holds them
    kf, vf = host(k[fa:fb, fheads]), host(v[fa:fb, fheads])
    say("varlen: inputs ready")
    w = torch.ones(H * D, dtype=BF16, device="cuda")
    cu_dev = torch.from_numpy(cu.astype(np.int32)).cuda()
    out, fs = la.prefill_varlen(q, k, v, g, w, cu_dev, return_final_state=True, check=True)
    torch.cuda.synchronize()
    # the longest sequence's state after its first lens - 1024 tokens, on every head
    say("varlen: state of the longest sequence before its last 1024 tokens")
    n0 = fw - fa
    fs_w = la.state(k[fa:fw].view(1, n0, H, D), v[fa:fw].view(1, n0, H, D), check=True)
    torch.cuda.synchronize()
    far_out, far_fs, fs_w = host(out[fw:fb]), host(fs[far:far + 1]), host(fs_w)
    # 2048-token chunks on the same pack: only the sampled sequences are kept
    say("varlen: chunk_tokens 2048")
    out_c, fs_c = la.prefill_varlen(q, k, v, g, w, cu_dev, return_final_state=True,
                                    chunk_tokens=2048, check=True)
    torch.cuda.synchronize()
    alt = {s: (host(out_c[int(cu[s]):int(cu[s + 1])]), host(fs_c[s:s + 1])) for s in picks}
    del q, k, v, g, out_c, fs_c
    wh = np.ones(H * D, np.float32)
    for s in picks + [mid]:
        a, b = int(cu[s]), int(cu[s + 1])
        ref, st = oracle.prefill(*wins[s], wh, return_state=True)
        check(host(out[a:b]), ref, BF16, "varlen sequence %d (%d tokens)" % (s, b - a))
        err = rel_state(host(fs[s:s + 1]), st)
        say("varlen sequence %d final state rel err %.2e" % (s, err))
        assert err < STATE_TOL
        if s in alt:
            check(alt[s][0], ref, BF16, "varlen sequence %d, 2048-token chunks" % s)
            assert rel_state(alt[s][1], st) < STATE_TOL
    # the longest sequence: states on the four heads, then the last window from
    # the GPU's state entering it
    st_w = None
    for a in range(0, n0, synth.CHUNK_TOKENS):
        b = min(n0, a + synth.CHUNK_TOKENS)
        st_w = oracle.state(kf[a:b], vf[a:b], init_state=st_w)
    err = rel_state(fs_w[:, fheads], st_w)
    say("varlen longest (%d tokens): state after %d tokens, heads %s, rel err %.2e"
        % (fb - fa, n0, fheads, err))
    assert err < STATE_TOL
    st_f = oracle.state(kf[n0:], vf[n0:], init_state=st_w)
    err = rel_state(far_fs[:, fheads], st_f)
    say("varlen longest: final state rel err %.2e" % err)
    assert err < STATE_TOL
    ref = oracle.prefill(*last, wh, init_state=fs_w)
    check(far_out, ref, BF16, "varlen longest, tokens [%d, %d) from the GPU state" % (n0, fb - fa))


@pytest.mark.slow
def test_prefill_1m_workload():
    N = 1 << 20
    T1 = N - 1024
    first = 2048
    picks = synth.pick_heads(4, H, synth.PREFILL_1M)
    say("prefill 1M: sampled heads", picks)
    q, k, v, g = (gpu_normal((N, H, D), 51 + t) for t in range(4))
    ids = (synth.Q, synth.K, synth.V, synth.G)
    # the four sampled heads' k and v on every token (kept for the oracle)
    kp = synth.block_tensor(synth.PREFILL_1M, synth.K, 0, N, picks, D, 1.0, threads=THREADS)
    vp = synth.block_tensor(synth.PREFILL_1M, synth.V, 0, N, picks, D, 1.0, threads=THREADS)
    put(k, slice(0, N), picks, kp)
    put(v, slice(0, N), picks, vp)
    say("prefill 1M: sampled heads' k, v ready")
    # every head on the first and the last window
    win = {}
    for a, b in ((0, first), (T1, N)):
        win[a] = [synth.block_tensor(synth.PREFILL_1M, t, a, b, range(H), D, 1.0, threads=THREADS)
                  for t in ids]
        for dst, x in zip((q, k, v, g), win[a]):
            put(dst, slice(a, b), range(H), x)
    w = torch.ones(H * D, dtype=BF16, device="cuda")
    wh = np.ones(H * D, np.float32)
    view = lambda t, n: t[:n].view(1, n, H, D)
    _, fs1 = la.prefill(*(view(t, T1) for t in (q, k, v, g)), w, return_final_state=True)
    out = la.prefill(*(view(t, N) for t in (q, k, v, g)), w)
    torch.cuda.synchronize()
    say("prefill 1M: GPU runs done")
    out_first, out_last = host(out[0, :first]), host(out[0, T1:])
    del q, k, v, g, out
    # state after T1 tokens on the sampled heads
    st = None
    for a in range(0, T1, synth.CHUNK_TOKENS):
        b = min(T1, a + synth.CHUNK_TOKENS)
        st = oracle.state(kp[a:b], vp[a:b], init_state=st)
    err = rel_state(host(fs1)[:, picks], st)
    say("prefill 1M: state after %d tokens, heads %s, rel err %.2e" % (T1, picks, err))
    assert err < STATE_TOL
    ref = oracle.prefill(*win[0], wh)
    check(out_first, ref, BF16, "prefill 1M tokens [0, %d)" % first)
    ref = oracle.prefill(*win[T1], wh, init_state=host(fs1))
    check(out_last, ref, BF16, "prefill 1M tokens [%d, %d) from the GPU state" % (T1, N))


@pytest.mark.slow
def test_layer_8k_hidden6144_workload():
    """lightning_attn_layer_prefill at the shape bench.py times: 8192 tokens,
    hidden 6144 (the model's), 64 heads x 128; x ~ N(0, 1), projections
    N(0, 1/fan_in), norm weight N(1, 0.02), all bf16 from seeded streams.
    Every output against the oracle's layer (fp64 products around the pinned
    prefill)."""
    N, hidden = 8192, 6144
    HD = H * D
    key = (synth.SEED, 92, 0)
    x = synth.normal(key + (0,), (N, hidden), bf16=True)
    wq = synth.normal(key + (1,), (4, hidden, HD), scale=1.0 / np.sqrt(hidden), bf16=True)
    w = synth.normal(key + (2,), (HD,), scale=0.02, mean=1.0, bf16=True)
    wo = synth.normal(key + (3,), (HD, hidden), scale=1.0 / np.sqrt(HD), bf16=True)
    say("layer 8K x hidden 6144: inputs ready")
    args = (dev(x, BF16).view(1, N, hidden), dev(wq, BF16), dev(w, BF16), dev(wo, BF16))
    outs = {}
    for gemm in ("mfma", "hipblaslt"):
        outs[gemm] = host(la.layer_prefill(*args, check=True, gemm=gemm)).reshape(N, hidden)
        torch.cuda.synchronize()
    del args
    say("layer 8K x hidden 6144: GPU done")
    ref = oracle.layer(x, wq, w, wo)
    for gemm, out in outs.items():
        check(out, ref, BF16, "layer 8192 tokens, hidden 6144, 64 heads, GEMM %s" % gemm)
