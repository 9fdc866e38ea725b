"""HIP path against the CPU oracle on seeded inputs (needs an MI355X).

Sizes are small enough for the fp64 oracle to finish in seconds while still
spanning several blocks, several chunks and a ragged tail; the full-size
workloads are in test_gpu_workloads.py.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check, dev, host, inputs, rel_state, say
import long_context_attn_amd as la

pytestmark = pytest.mark.gpu

# Final-state bound, relative to max|state|.  bf16 inputs: the MFMA path
# multiplies bf16-rounded SiLU(k) and SiLU(v), each product off by at most
# 2 * 2^-9 relative, so a sum of such products is within 2^-8 ~ 3.9e-3 of the
# exact state.  fp32 inputs: fp32 arithmetic throughout.
STATE_TOL = {torch.float32: 1e-5, torch.bfloat16: 4e-3}


def plan_error(ws):
    """Error code the kernels leave in the workspace (0 = ok), through the C ABI."""
    return la.workspace_status(ws)[0]


def run_prefill(q, k, v, g, w, B, dtype, block, chunk=0, init=None, eps=1e-6):
    T, H, D = q.shape
    N = T // B
    qd, kd, vd, gd = (dev(a, dtype).view(B, N, H, D) for a in (q, k, v, g))
    wd = dev(w, dtype)
    initd = None if init is None else torch.from_numpy(init.astype(np.float32)).cuda()
    ws = torch.empty(la.prefill_workspace_size(T, B, H, D, block, chunk, dtype), dtype=torch.uint8,
                     device="cuda")
    out, fs = la.prefill(qd, kd, vd, gd, wd, block=block, eps=eps, initial_state=initd,
                         return_final_state=True, chunk_tokens=chunk, workspace=ws)
    torch.cuda.synchronize()
    assert plan_error(ws) == 0
    return out.view(T, H, D), fs


def oracle_prefill(q, k, v, g, w, B, init=None, eps=1e-6):
    T = q.shape[0]
    seg = np.arange(B + 1) * (T // B)
    return oracle.prefill(q, k, v, g, w, cu_seqlens=seg, eps=eps, init_state=init,
                          return_state=True)


def test_tiny_fp32_workload():
    """B=1, 2 heads, head_dim 64, 256 tokens, block 32, fp32, N(0,1), weight 1."""
    H, D, N = 2, 64, 256
    q, k, v, g, w = inputs(N, H, D, "unit", bf16=False, key=1)
    ref, st = oracle_prefill(q, k, v, g, w, 1)
    for chunk in (0, 32, 96, 256):
        say("tiny fp32 chunk", chunk)
        out, fs = run_prefill(q, k, v, g, w, 1, torch.float32, 32, chunk)
        check(out, ref, torch.float32, "tiny fp32 chunk=%d" % chunk)
        assert rel_state(host(fs), st) < STATE_TOL[torch.float32]


@pytest.mark.parametrize("D,block", [(16, 16), (32, 32), (64, 64), (128, 32), (128, 64)])
def test_fp32_shapes_ragged_with_state(D, block):
    B, N, H = 2, 301, 3
    q, k, v, g, w = inputs(B * N, H, D, "unit", bf16=False, key=2)
    init = np.random.default_rng(D).standard_normal((B, H, D, D)).astype(np.float32)
    ref, st = oracle_prefill(q, k, v, g, w, B, init=init)
    say("fp32 D", D, "block", block)
    out, fs = run_prefill(q, k, v, g, w, B, torch.float32, block, 2 * block, init=init)
    check(out, ref, torch.float32, "fp32 D=%d block=%d" % (D, block))
    assert rel_state(host(fs), st) < STATE_TOL[torch.float32]


@pytest.mark.parametrize("D,block,dist", [(64, 32, "unit"), (64, 64, "minimax"),
                                          (128, 64, "unit"), (128, 64, "minimax"),
                                          (128, 32, "unit")])
def test_bf16_ragged(D, block, dist):
    B, N, H = 2, 1000, 4
    q, k, v, g, w = inputs(B * N, H, D, dist, key=3)
    ref, st = oracle_prefill(q, k, v, g, w, B)
    # 0 picks the chunk length automatically (128 tokens at 4 heads)
    for chunk in (0, block, 4 * block):
        say("bf16 D", D, "block", block, dist, "chunk", chunk)
        out, fs = run_prefill(q, k, v, g, w, B, torch.bfloat16, block, chunk)
        check(out, ref, torch.bfloat16, "bf16 D=%d block=%d %s chunk=%d" % (D, block, dist, chunk))
        assert rel_state(host(fs), st) < STATE_TOL[torch.bfloat16]


def test_bf16_more_heads_than_cus():
    """bf16, head_dim 128, block 64 with more heads than the device has CUs:
    the fused walk's cross-head exchange needs every head of a chunk resident
    at once, so such calls run the portable kernels (walk, then the separate
    norm); they must still match the oracle, with a ragged tail and a final
    state."""
    H = torch.cuda.get_device_properties(0).multi_processor_count + 4
    N, D = 130, 128
    q, k, v, g, w = inputs(N, H, D, "unit", key=13)
    ref, st = oracle_prefill(q, k, v, g, w, 1)
    say("bf16 with", H, "heads (more than the CUs)")
    out, fs = run_prefill(q, k, v, g, w, 1, torch.bfloat16, 64, 0)
    check(out, ref, torch.bfloat16, "bf16 H=%d" % H)
    assert rel_state(host(fs), st) < STATE_TOL[torch.bfloat16]


@pytest.mark.parametrize("dtype,D,block", [(torch.float32, 64, 32), (torch.bfloat16, 128, 64)])
def test_varlen_packed(dtype, D, block):
    lens = [0, 1, 63, 64, 65, 130, 700, 0, 3, 2 * block + 7]
    seg = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, H = int(seg[-1]), 3
    q, k, v, g, w = inputs(T, H, D, "unit", bf16=dtype == torch.bfloat16, key=4)
    init = np.random.default_rng(5).standard_normal((len(lens), H, D, D)).astype(np.float32)
    ref, st = oracle.prefill(q, k, v, g, w, cu_seqlens=seg, init_state=init, return_state=True)
    cu = torch.from_numpy(seg.astype(np.int32)).cuda()
    for chunk in (0, block, 2 * block):
        say("varlen", dtype, "chunk", chunk)
        ws = torch.empty(la.prefill_workspace_size(T, len(lens), H, D, block, chunk, dtype),
                         dtype=torch.uint8, device="cuda")
        out, fs = la.prefill_varlen(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(g, dtype),
                                    dev(w, dtype), cu, block=block,
                                    initial_state=torch.from_numpy(init).cuda(),
                                    return_final_state=True, chunk_tokens=chunk, workspace=ws)
        torch.cuda.synchronize()
        assert plan_error(ws) == 0
        check(out, ref, dtype, "varlen chunk=%d" % chunk)
        assert rel_state(host(fs), st) < STATE_TOL[dtype]


@pytest.mark.parametrize("dtype,D,S", [(torch.float32, 64, 6), (torch.bfloat16, 128, 6),
                                       (torch.bfloat16, 32, 6), (torch.float32, 64, 300),
                                       (torch.bfloat16, 128, 260)])
def test_decode_steps(dtype, D, S):
    """S >= the CU count (256) takes the one-workgroup-per-sequence kernel with
    the norm fused; fewer sequences take the pair loop and the norm kernel."""
    H, L = 4, 40
    bf = dtype == torch.bfloat16
    q, k, v, g, w = inputs(S * L, H, D, "unit", bf16=bf, key=6)
    seg = np.arange(S + 1) * L
    st0 = oracle.state(k, v, cu_seqlens=seg).astype(np.float32)  # fp32 initial state, both sides
    state_ref = st0.astype(np.float64)
    state_gpu = torch.from_numpy(st0).cuda()
    wd = dev(w, dtype)
    for step in range(3):
        qs, ks, vs, gs = (inputs(S, H, D, "unit", bf16=bf, key=100 + step)[i] for i in range(4))
        ref, state_ref = oracle.decode(qs, ks, vs, gs, w, state_ref)
        say("decode", dtype, "D", D, "S", S, "step", step)
        out = la.decode(dev(qs, dtype), dev(ks, dtype), dev(vs, dtype), dev(gs, dtype), wd,
                        state_gpu)
        torch.cuda.synchronize()
        check(out, ref, dtype, "decode step %d" % step)
        assert rel_state(host(state_gpu), state_ref) < 1e-6


@pytest.mark.parametrize("chunk", [0, 64])
def test_decode_after_prefill_on_gpu(chunk):
    """GPU prefill of L tokens then m GPU decode steps == GPU prefill of L+m."""
    H, D, L, m = 4, 128, 200, 3
    q, k, v, g, w = inputs(L + m, H, D, "unit", key=8)
    dt = torch.bfloat16
    full, _ = run_prefill(q, k, v, g, w, 1, dt, 64, chunk)
    _, st = run_prefill(q[:L], k[:L], v[:L], g[:L], w, 1, dt, 64, chunk)
    st = st.contiguous()
    ref = oracle.prefill(q, k, v, g, w)
    for i in range(m):
        t = L + i
        say("decode-after-prefill", i)
        o = la.decode(*(dev(a[t:t + 1], dt) for a in (q, k, v, g)), dev(w, dt), st.view(1, H, D, D))
        torch.cuda.synchronize()
        check(o[0], ref[t], dt, "decode-after-prefill token %d" % t)
        check(o[0], host(full[t]), dt, "decode vs prefill row %d" % t)


def test_empty_and_repeatable():
    H, D = 2, 128
    dt = torch.bfloat16
    init = torch.randn(1, H, D, D, device="cuda")
    z = torch.empty(1, 0, H, D, dtype=dt, device="cuda")
    w = torch.ones(H * D, dtype=dt, device="cuda")
    say("empty prefill")
    out, fs = la.prefill(z, z, z, z, w, initial_state=init, return_final_state=True)
    torch.cuda.synchronize()
    assert out.numel() == 0 and torch.equal(fs, init)
    q, k, v, g, w = inputs(777, H, D, "unit", key=9)
    for chunk in (0, 128):
        say("repeatability, chunk", chunk)
        a, sa = run_prefill(q, k, v, g, w, 1, dt, 64, chunk)
        b, sb = run_prefill(q, k, v, g, w, 1, dt, 64, chunk)
        assert torch.equal(a, b) and torch.equal(sa, sb)


@pytest.mark.parametrize("chunk", [0, 64])
def test_invalid_cu_seqlens_reported(chunk):
    """cu_seqlens that does not end at total_tokens: the plan records error 1 in
    the workspace header, the launch finishes, and a valid call on the same
    workspace afterwards is correct again."""
    H, D, T = 4, 128, 300
    q, k, v, g, w = inputs(T, H, D, "unit", key=11)
    dt = torch.bfloat16
    args = [dev(a, dt) for a in (q, k, v, g, w)]
    bad = torch.tensor([0, 100, 250], dtype=torch.int32, device="cuda")  # ends at 250, not 300
    ws = torch.empty(la.prefill_workspace_size(T, 2, H, D, 64, chunk, dt), dtype=torch.uint8,
                     device="cuda")
    say("invalid cu_seqlens, chunk", chunk)
    la.prefill_varlen(*args, bad, chunk_tokens=chunk, workspace=ws)
    torch.cuda.synchronize()
    assert la.workspace_status(ws) == (1, 0, 0, 0)
    # the binding raises on it when asked (check=True, or LA_DEBUG=1)
    with pytest.raises(la.LightningAttnDeviceError, match="cu_seqlens"):
        la.prefill_varlen(*args, bad, chunk_tokens=chunk, workspace=ws, check=True)
    good = torch.tensor([0, 100, 300], dtype=torch.int32, device="cuda")
    out = la.prefill_varlen(*args, good, chunk_tokens=chunk, workspace=ws)
    torch.cuda.synchronize()
    assert plan_error(ws) == 0
    ref = oracle.prefill(q, k, v, g, w, cu_seqlens=np.array([0, 100, 300]))
    check(out, ref, dt, "after an invalid call, chunk %d" % chunk)
