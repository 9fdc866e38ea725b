"""Seeded synthetic inputs for the Lightning Attention layer.

This module only draws numbers: it holds none of the layer's arithmetic, and
both the GPU path and the CPU oracle are fed from it.  Every stream is
numpy ``Generator(PCG64(SeedSequence(key)))`` with ``key = [2025, workload,
tensor, chunk]``, so any piece of any workload can be regenerated on its own
(the 1M-token workloads are generated chunk by chunk, never whole).

Values are ``standard_normal(float32)`` times a scale (in fp32), then rounded
to bf16 with round-to-nearest-even when the workload is bf16.  Arrays are
returned as float32 holding exactly representable values, so converting them
to torch bf16 or to float64 is exact.

Workload distributions (the layer's inputs are pre-activation q/k/v/gate):
  * "unit":    q, k, v, gate ~ N(0, 1), norm weight all ones;
  * "minimax": q, k, v ~ N(0, 1)/sqrt(D), gate ~ N(0, 1), weight ~ N(1, 0.02).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED = 2025
CHUNK_TOKENS = 65536
BLOCK_TOKENS = 1024

# tensor ids inside a workload key
Q, K, V, G, W, LENGTHS, HEAD_PICK, S0_K, S0_V = range(9)

# workload ids: 1 tiny fp32 prefill, 2 8K prefill, 3 decode, 4 1M varlen, 5 1M prefill
TINY_FP32, PREFILL_8K, DECODE, VARLEN_1M, PREFILL_1M = 1, 2, 3, 4, 5


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite values never wrap in uint32: the largest finite pattern plus 0x8000 stays below 2^32
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def stream(key, n: int) -> np.ndarray:
    """First n standard normals (float32) of the stream named by key."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))
    return g.standard_normal(n, dtype=np.float32)


def normal(key, shape, scale: float = 1.0, mean: float = 0.0, bf16: bool = True) -> np.ndarray:
    """Array of the given shape from one stream: mean + scale * N(0,1), fp32 math."""
    n = int(np.prod(shape)) if len(shape) else 1
    x = stream(key, n).reshape(shape)
    if scale != 1.0:
        x = x * np.float32(scale)
    if mean != 0.0:
        x = x + np.float32(mean)
    return round_bf16(x) if bf16 else x.astype(np.float32)


def scales(dist: str, D: int):
    """(q/k/v scale, gate scale, weight mean, weight std) for a distribution."""
    if dist == "unit":
        return 1.0, 1.0, 1.0, 0.0
    if dist == "minimax":
        return 1.0 / math.sqrt(D), 1.0, 1.0, 0.02
    raise ValueError("unknown distribution %r" % dist)


def token_tensor(workload: int, tensor: int, t0: int, t1: int, H: int, D: int, scale: float,
                 bf16: bool = True, threads: int = 1) -> np.ndarray:
    """Tokens [t0, t1) of a [T, H, D] activation, drawn per 65,536-token chunk.

    Chunk c of the tensor is the stream [2025, workload, tensor, c]; its first
    (t - 65536 c) * H * D values belong to tokens before t.
    """
    out = np.empty((t1 - t0, H, D), np.float32)
    HD = H * D
    pieces = []
    c = t0 // CHUNK_TOKENS
    while c * CHUNK_TOKENS < t1:
        a = max(t0, c * CHUNK_TOKENS)
        b = min(t1, (c + 1) * CHUNK_TOKENS)
        pieces.append((c, a, b))
        c += 1

    def fill(p):
        c, a, b = p
        base = c * CHUNK_TOKENS
        x = stream((SEED, workload, tensor, c), (b - base) * HD)[(a - base) * HD:]
        x = x.reshape(b - a, H, D)
        if scale != 1.0:
            x = x * np.float32(scale)
        out[a - t0:b - t0] = round_bf16(x) if bf16 else x

    if threads > 1 and len(pieces) > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, pieces))
    else:
        for p in pieces:
            fill(p)
    return out


def block_tensor(workload: int, tensor: int, t0: int, t1: int, heads, D: int, scale: float,
                 bf16: bool = True, threads: int = 1) -> np.ndarray:
    """Tokens [t0, t1) of the given heads of a [T, H, D] activation whose
    values are drawn per (1024-token block, head).

    Block j of head h is the stream [2025, workload, tensor, j, h] of 1024 * D
    values, so any window of tokens or subset of heads can be drawn without
    drawing the rest: the full-size parity tests use this for the 1M-token
    workloads.  Returns [t1 - t0, len(heads), D].
    """
    heads = list(heads)
    out = np.empty((t1 - t0, len(heads), D), np.float32)
    jobs = [(j, i, h) for j in range(t0 // BLOCK_TOKENS, (t1 + BLOCK_TOKENS - 1) // BLOCK_TOKENS)
            for i, h in enumerate(heads)]

    def fill(job):
        j, i, h = job
        base = j * BLOCK_TOKENS
        a, b = max(t0, base), min(t1, base + BLOCK_TOKENS)
        x = stream((SEED, workload, tensor, j, h), (b - base) * D)[(a - base) * D:]
        x = x.reshape(b - a, D)
        if scale != 1.0:
            x = x * np.float32(scale)
        out[a - t0:b - t0, i] = round_bf16(x) if bf16 else x

    if threads > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, jobs, chunksize=max(1, len(jobs) // (8 * threads))))
    else:
        for job in jobs:
            fill(job)
    return out


def layer_inputs(workload: int, T: int, H: int, D: int, dist: str, bf16: bool = True,
                 t0: int = 0, threads: int = 1):
    """q, k, v, gate for tokens [t0, t0+T) and the norm weight [H*D]."""
    s, gs, wm, ws = scales(dist, D)
    q = token_tensor(workload, Q, t0, t0 + T, H, D, s, bf16, threads)
    k = token_tensor(workload, K, t0, t0 + T, H, D, s, bf16, threads)
    v = token_tensor(workload, V, t0, t0 + T, H, D, s, bf16, threads)
    g = token_tensor(workload, G, t0, t0 + T, H, D, gs, bf16, threads)
    w = norm_weight(workload, H, D, dist, bf16)
    return q, k, v, g, w


def norm_weight(workload: int, H: int, D: int, dist: str, bf16: bool = True) -> np.ndarray:
    _, _, wm, ws = scales(dist, D)
    if ws == 0.0:
        return np.full(H * D, np.float32(wm), np.float32)
    return normal((SEED, workload, W, 0), (H * D,), scale=ws, mean=wm, bf16=bf16)


def varlen_lengths(total: int, lo: int = 1024, hi: int = 131072, workload: int = VARLEN_1M):
    """Sequence lengths drawn log-uniform in [lo, hi) until they reach `total`.

    L = floor(exp(U[ln lo, ln hi))); drawing stops once the running sum reaches
    `total` and the last length is cut so the sum is exactly `total`.
    """
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, workload, LENGTHS, 0])))
    lens = []
    acc = 0
    while acc < total:
        L = int(math.floor(math.exp(g.uniform(math.log(lo), math.log(hi)))))
        L = min(L, total - acc)
        lens.append(L)
        acc += L
    return lens


def cu_seqlens(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int64)


def decode_prefix_lengths(nseq: int, lo: int = 1024, hi: int = 32768, workload: int = DECODE):
    """Per-sequence prefill length for the decode workload's initial state, U{lo..hi}."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, workload, LENGTHS, 0])))
    return [int(x) for x in g.integers(lo, hi, size=nseq, endpoint=True)]


def decode_prefix_kv(seq: int, L: int, H: int, D: int, dist: str = "unit",
                     workload: int = DECODE):
    """k, v [L, H, D] of sequence `seq`'s prefill that defines its initial state."""
    s, _, _, _ = scales(dist, D)
    k = normal((SEED, workload, S0_K, seq), (L, H, D), scale=s)
    v = normal((SEED, workload, S0_V, seq), (L, H, D), scale=s)
    return k, v


def decode_step_inputs(step: int, nseq: int, H: int, D: int, dist: str = "unit",
                       workload: int = DECODE):
    """Fresh q, k, v, gate [nseq, H, D] for decode step `step`."""
    s, gs, _, _ = scales(dist, D)
    return tuple(normal((SEED, workload, t, 1000 + step), (nseq, H, D), scale=(gs if t == G else s))
                 for t in (Q, K, V, G))


def pick(n: int, pool: int, workload: int, what: int = 0) -> list:
    """n distinct indices in [0, pool) chosen by the seeded stream of a workload."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, workload, HEAD_PICK, what])))
    return sorted(int(h) for h in g.choice(pool, size=n, replace=False))


def pick_heads(n: int, H: int, workload: int) -> list:
    """n distinct heads chosen by the seeded stream of a workload."""
    return pick(n, H, workload, 0)
