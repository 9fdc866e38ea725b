"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph on ROCm).

Every call enqueues kernels only on the caller's stream, with no memset, no
allocation and no host synchronisation, so a prefill followed by decode steps
can be captured once and replayed.  Each replay here runs on new inputs copied
into the captured buffers, with eager work and synchronisations in between,
and must equal the eager calls on the same inputs bit for bit; the first
replay is also held to the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check, dev, host, inputs, say
import long_context_attn_amd as la

pytestmark = pytest.mark.gpu


def test_prefill_and_decode_steps_in_one_graph():
    B, N, H, D, steps = 2, 300, 4, 128, 3
    dt = torch.bfloat16
    draws = []
    for key in range(3):  # three sets of inputs: one per replay
        q, k, v, g, w = inputs(B * N + B * steps, H, D, "unit", key=40 + key)
        draws.append((q, k, v, g, w))
    w = dev(draws[0][4], dt)
    # captured buffers: the prefill's [B, N, H, D] inputs and each decode step's [B, H, D]
    xq, xk, xv, xg = (torch.empty(B, N, H, D, dtype=dt, device="cuda") for _ in range(4))
    sq, sk, sv, sg = (torch.empty(steps, B, H, D, dtype=dt, device="cuda") for _ in range(4))
    out = torch.empty(B, N, H, D, dtype=dt, device="cuda")
    outs = torch.empty(steps, B, H, D, dtype=dt, device="cuda")
    state = torch.empty(B, H, D, D, dtype=torch.float32, device="cuda")
    ws = torch.empty(la.prefill_workspace_size(B * N, B, H, D, 64, 0, dt), dtype=torch.uint8,
                     device="cuda")
    dws = torch.empty(la.decode_workspace_size(B, H, D), dtype=torch.uint8, device="cuda")

    def fill(i):
        q, k, v, g, _ = draws[i]
        pre = lambda a: dev(a[:B * N], dt).view(B, N, H, D)
        step = lambda a: dev(a[B * N:], dt).view(steps, B, H, D)
        for dst, a in ((xq, q), (xk, k), (xv, v), (xg, g)):
            dst.copy_(pre(a))
        for dst, a in ((sq, q), (sk, k), (sv, v), (sg, g)):
            dst.copy_(step(a))

    def layer_calls():
        la.prefill(xq, xk, xv, xg, w, out=out, return_final_state=True, final_state=state,
                   workspace=ws)
        for s in range(steps):
            la.decode(sq[s], sk[s], sv[s], sg[s], w, state, out=outs[s], workspace=dws)

    # eager results for every set of inputs
    eager = []
    for i in range(len(draws)):
        fill(i)
        layer_calls()
        torch.cuda.synchronize()
        eager.append((out.clone(), outs.clone(), state.clone()))

    # capture once (after a warm-up on a side stream, as torch asks), then replay
    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer_calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer_calls()
    torch.cuda.synchronize()
    for rep in range(2):
        for i in (1, 0, 2):
            say("graph replay %d on input set %d" % (rep, i))
            fill(i)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager[i][0]), ("prefill out", rep, i)
            assert torch.equal(outs, eager[i][1]), ("decode outs", rep, i)
            assert torch.equal(state, eager[i][2]), ("state", rep, i)
            # eager work in between replays
            torch.ones(1 << 20, device="cuda").sum().item()

    # and the replayed results against the oracle (input set 0)
    q, k, v, g, wn = draws[0]
    seg = np.arange(B + 1) * N
    ref, st = oracle.prefill(q[:B * N], k[:B * N], v[:B * N], g[:B * N], wn, cu_seqlens=seg,
                             return_state=True)
    check(eager[0][0].view(B * N, H, D), ref, dt, "prefill under a graph")
    stn = st.copy()
    for s in range(steps):
        a = B * N + s * B
        r, stn = oracle.decode(q[a:a + B], k[a:a + B], v[a:a + B], g[a:a + B], wn, stn)
        check(eager[0][1][s], r, dt, "decode step %d under a graph" % s)
