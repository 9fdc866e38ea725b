"""State-only calls (lightning_attn_state / _varlen) against the CPU oracle,
and the two-pass split of one prefill along its sequence that they exist for
(needs an MI355X).

The split follows the sequence-parallel scheme the MiniMax-Text-01 summary
page lists (LASP+): each part's state sum, an exclusive prefix over the parts,
then a prefill of each part started from its prefix.  Its outputs must match
the oracle's prefill of the whole sequence.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check, dev, host, inputs, rel_state, say
import long_context_attn_amd as la

pytestmark = pytest.mark.gpu

# see test_gpu_parity.py: bf16 states are within 2^-8 relative of the exact sum
STATE_TOL = {torch.float32: 1e-5, torch.bfloat16: 4e-3}
# bf16 D=128 block 64 runs the MFMA chunk-state kernel, the others the fp32 one
CASES = [(torch.bfloat16, 128, 64), (torch.bfloat16, 64, 32), (torch.float32, 64, 32),
         (torch.float32, 128, 64)]


def plan_error(ws):
    return la.workspace_status(ws)[0]


@pytest.mark.parametrize("dtype,D,block", CASES)
def test_state_batch(dtype, D, block):
    B, N, H = 2, 1000, 3
    bf16 = dtype == torch.bfloat16
    _, k, v, _, _ = inputs(B * N, H, D, "unit", bf16=bf16, key=11)
    init = np.random.default_rng(12).standard_normal((B, H, D, D)).astype(np.float32)
    seg = np.arange(B + 1) * N
    ref0 = oracle.state(k, v, cu_seqlens=seg)
    ref1 = oracle.state(k, v, cu_seqlens=seg, init_state=init)
    kd, vd = (dev(a, dtype).view(B, N, H, D) for a in (k, v))
    for chunk in (0, block, 3 * block, 1024):
        say("state", dtype, "D", D, "block", block, "chunk", chunk)
        ws = torch.empty(la.state_workspace_size(B * N, B, H, D, block, chunk, dtype),
                         dtype=torch.uint8, device="cuda")
        fs = la.state(kd, vd, block=block, chunk_tokens=chunk, workspace=ws)
        torch.cuda.synchronize()
        assert plan_error(ws) == 0
        assert rel_state(host(fs), ref0) < STATE_TOL[dtype]
        # in place: the final state overwrites the initial one
        st = torch.from_numpy(init).cuda()
        out = la.state(kd, vd, block=block, initial_state=st, final_state=st, chunk_tokens=chunk)
        torch.cuda.synchronize()
        assert out.data_ptr() == st.data_ptr()
        assert rel_state(host(st), ref1) < STATE_TOL[dtype]


@pytest.mark.parametrize("dtype,D,block", CASES[:1] + CASES[2:3])
def test_state_varlen_with_empty_sequences(dtype, D, block):
    lens = [0, 1, 63, 64, 65, 700, 0, 3, 2 * block + 7, 0]
    seg = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, H = int(seg[-1]), 2
    _, k, v, _, _ = inputs(T, H, D, "minimax", bf16=dtype == torch.bfloat16, key=13)
    init = np.random.default_rng(14).standard_normal((len(lens), H, D, D)).astype(np.float32)
    ref = oracle.state(k, v, cu_seqlens=seg, init_state=init)
    cu = torch.from_numpy(seg.astype(np.int32)).cuda()
    for chunk in (0, block, 2 * block):
        say("state varlen", dtype, "chunk", chunk)
        fs = la.state_varlen(dev(k, dtype), dev(v, dtype), cu, block=block,
                             initial_state=torch.from_numpy(init).cuda(), chunk_tokens=chunk)
        torch.cuda.synchronize()
        got = host(fs)
        assert rel_state(got, ref) < STATE_TOL[dtype]
        # an empty sequence's final state is its initial state, bit for bit
        for s, L in enumerate(lens):
            if L == 0:
                assert np.array_equal(got[s], init[s])


@pytest.mark.parametrize("dtype,D,block", [(torch.bfloat16, 128, 64), (torch.float32, 64, 32)])
def test_sequence_split_prefill(dtype, D, block):
    """One 2000-token sequence cut into parts of uneven lengths (not multiples
    of the block): state-only pass over every part, exclusive prefix of the part
    states on the host in fp64, prefill of each part from its prefix."""
    N, H = 2000, 4
    q, k, v, g, w = inputs(N, H, D, "minimax", bf16=dtype == torch.bfloat16, key=15)
    ref, st = oracle.prefill(q, k, v, g, w, return_state=True)
    cuts = [0, 517, 1024, 1100, 2000]
    P = len(cuts) - 1
    kd, vd = dev(k, dtype), dev(v, dtype)
    cu = torch.tensor(cuts, dtype=torch.int32, device="cuda")
    say("split prefill: part states", dtype)
    parts = host(la.state_varlen(kd, vd, cu, block=block)).astype(np.float64)
    prefix = np.zeros((H, D, D))
    outs = []
    for p in range(P):
        a, b = cuts[p], cuts[p + 1]
        sl = [dev(x[a:b], dtype).view(1, b - a, H, D) for x in (q, k, v, g)]
        init = torch.from_numpy(prefix[None].astype(np.float32)).cuda()
        say("split prefill: part", p, "tokens", a, b)
        out, fs = la.prefill(*sl, dev(w, dtype), block=block, initial_state=init,
                             return_final_state=True)
        torch.cuda.synchronize()
        outs.append(host(out).reshape(b - a, H, D))
        prefix = prefix + parts[p]
        # each part's prefill ends in the state the prefix reaches after it
        assert rel_state(host(fs)[0], prefix) < 2 * STATE_TOL[dtype]
    check(np.concatenate(outs), ref, dtype, "sequence split into %d parts" % P)
    assert rel_state(prefix, st[0]) < STATE_TOL[dtype]


def test_state_empty_calls():
    k = torch.empty(0, 2, 64, dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    init = torch.randn(3, 2, 64, 64, device="cuda")
    fs = la.state_varlen(k, k, cu, block=32, initial_state=init)
    torch.cuda.synchronize()
    assert torch.equal(fs, init)
    fs = la.state(torch.empty(2, 0, 2, 64, dtype=torch.bfloat16, device="cuda"),
                  torch.empty(2, 0, 2, 64, dtype=torch.bfloat16, device="cuda"), block=32)
    torch.cuda.synchronize()
    assert torch.count_nonzero(fs) == 0
