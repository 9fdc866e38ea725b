"""The layer with its projections (lightning_attn_layer_prefill) against the
oracle (needs an MI355X).

The oracle multiplies in float64 (x Wq, x Wk, x Wv, x Wg, then the attention
output by Wo) around its pinned prefill.  On the GPU the projections are bf16
GEMMs with fp32 accumulation, either the library's own MFMA kernel (SiLU on
q, k, v and the logistic function on the gate in its epilogue) or hipBLASLt
(SiLU in the q, k, v epilogues, the gate's sigmoid in the attention); the
attention reads one bf16 rounding of each activated operand, as the bf16
prefill does, and the result is held to the bf16 bar.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check, dev, host, rel_state, say
import long_context_attn_amd as la
from long_context_attn_amd import synth

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def layer_inputs(T, hidden, H, key):
    D = 128
    HD = H * D
    x = synth.normal((synth.SEED, 91, key, 0), (T, hidden), bf16=True)
    wq = synth.normal((synth.SEED, 91, key, 1), (4, hidden, HD), scale=1.0 / np.sqrt(hidden),
                      bf16=True)
    w = synth.normal((synth.SEED, 91, key, 2), (HD,), scale=0.02, mean=1.0, bf16=True)
    wo = synth.normal((synth.SEED, 91, key, 3), (HD, hidden), scale=1.0 / np.sqrt(HD), bf16=True)
    return x, wq, w, wo


@pytest.mark.parametrize("gemm", ["mfma", "hipblaslt"])
@pytest.mark.parametrize("B,N,hidden,H", [(2, 300, 256, 2), (1, 1100, 512, 4), (3, 64, 384, 1),
                                          (1, 700, 320, 3)])
def test_layer_against_oracle(B, N, hidden, H, gemm):
    D = 128
    T = B * N
    x, wq, w, wo = layer_inputs(T, hidden, H, key=31 + H)
    init = np.random.default_rng(H).standard_normal((B, H, D, D)).astype(np.float32) * 0.1
    seg = np.arange(B + 1) * N
    ref, st = oracle.layer(x, wq, w, wo, cu_seqlens=seg, init_state=init, return_state=True)
    say("layer B", B, "N", N, "hidden", hidden, "H", H, "gemm", gemm)
    out, fs = la.layer_prefill(dev(x, BF16).view(B, N, hidden), dev(wq, BF16), dev(w, BF16),
                               dev(wo, BF16), initial_state=torch.from_numpy(init).cuda(),
                               return_final_state=True, gemm=gemm, check=True)
    torch.cuda.synchronize()
    check(host(out).reshape(T, hidden), ref, BF16,
          "layer B=%d N=%d hidden=%d H=%d gemm=%s" % (B, N, hidden, H, gemm))
    err = rel_state(host(fs), st)
    say("layer final state rel err %.2e" % err)
    assert err < 8e-3


@pytest.mark.parametrize("gemm", ["mfma", "hipblaslt"])
def test_layer_matches_prefill_on_projected_inputs(gemm):
    """The layer's attention equals lightning_attn_prefill run on the same
    projected inputs: with Wo = I the two outputs agree to bf16 rounding."""
    B, N, H, D = 1, 500, 2, 128
    HD = hidden = H * D
    x, wq, w, _ = layer_inputs(B * N, hidden, H, key=40)
    eye = np.eye(HD, dtype=np.float32)
    out = la.layer_prefill(dev(x, BF16).view(B, N, hidden), dev(wq, BF16), dev(w, BF16),
                           dev(eye, BF16), gemm=gemm)
    torch.cuda.synchronize()
    xs = dev(x, BF16).float()
    proj = [(xs @ dev(wq[i], BF16).float()) for i in range(4)]
    q, k, v, g = (p.to(BF16).view(B, N, H, D) for p in proj)
    ref = la.prefill(q, k, v, g, dev(w, BF16))
    torch.cuda.synchronize()
    emax, emean = oracle.compare(host(out).reshape(N, HD), host(ref).reshape(N, HD))
    say("layer vs prefill on projected inputs: e_max %.2e e_mean %.2e" % (emax, emean))
    assert emax < 2e-2 and emean < 2e-3


def test_layer_gemm_backends_agree():
    """The library's GEMM and hipBLASLt on the same layer inputs (ragged token
    count, hidden a multiple of 64 but not of the 256-wide tiles): both
    round the same fp32 products to bf16, so they agree to bf16 rounding."""
    B, N, hidden, H = 2, 517, 448, 2
    x, wq, w, wo = layer_inputs(B * N, hidden, H, key=44)
    args = (dev(x, BF16).view(B, N, hidden), dev(wq, BF16), dev(w, BF16), dev(wo, BF16))
    a = la.layer_prefill(*args, gemm="mfma")
    b = la.layer_prefill(*args, gemm="hipblaslt")
    torch.cuda.synchronize()
    emax, emean = oracle.compare(host(a).reshape(B * N, hidden), host(b).reshape(B * N, hidden))
    say("layer, MFMA GEMM vs hipBLASLt: e_max %.2e e_mean %.2e" % (emax, emean))
    assert emax < 2e-2 and emean < 2e-3
