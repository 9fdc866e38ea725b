"""Helpers shared by the GPU tests: seeded inputs on the device, oracle
comparison with the tolerances of the layer's correctness bar."""
import sys

import numpy as np
import torch

import oracle
from long_context_attn_amd import synth

# correctness bar, measured after the RMSNorm * gate epilogue, relative to max|out_ref|
TOL = {torch.float32: (1e-4, None), torch.bfloat16: (2e-2, 2e-3)}


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype).contiguous()


def host(t):
    return t.detach().float().cpu().numpy()


def check(out_gpu, out_ref, dtype, what=""):
    emax, emean = oracle.compare(host(out_gpu) if torch.is_tensor(out_gpu) else out_gpu, out_ref)
    tmax, tmean = TOL[dtype]
    say("%s e_max=%.3e e_mean=%.3e (bar %.0e / %s)" % (what, emax, emean, tmax, tmean))
    assert emax <= tmax, (what, emax)
    if tmean is not None:
        assert emean <= tmean, (what, emean)
    return emax, emean


def rel_state(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def inputs(T, H, D, dist="unit", bf16=True, key=7, w_dist=None):
    """Small seeded activations [T, H, D] (one stream per tensor) and weight."""
    s, gs, wm, ws = synth.scales(dist, D)
    q = synth.normal((synth.SEED, 90, key, 0), (T, H, D), scale=s, bf16=bf16)
    k = synth.normal((synth.SEED, 90, key, 1), (T, H, D), scale=s, bf16=bf16)
    v = synth.normal((synth.SEED, 90, key, 2), (T, H, D), scale=s, bf16=bf16)
    g = synth.normal((synth.SEED, 90, key, 3), (T, H, D), scale=gs, bf16=bf16)
    if ws == 0.0:
        w = np.full(H * D, np.float32(wm))
    else:
        w = synth.normal((synth.SEED, 90, key, 4), (H * D,), scale=ws, mean=wm, bf16=bf16)
    return q, k, v, g, w
