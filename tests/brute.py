"""Independent left-product statement of the layer, used only to pin the oracle.

Y = (Q~ K~^T (.) M) V~ + Q~ S0 per segment and head, M lower triangular with
the diagonal (quadratic in length, so tiny inputs only); sigmoid from scipy.
It deliberately shares nothing with oracle/la_oracle.c, which walks tokens
through the D x D state instead.
"""
import numpy as np
from scipy.special import expit


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * expit(x)


def attention(q, k, v, seg, init=None):
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    T, H, D = q.shape
    qs, ks, vs = silu(q), silu(k), silu(v)
    y = np.zeros((T, H, D))
    for s in range(len(seg) - 1):
        a, b = int(seg[s]), int(seg[s + 1])
        for h in range(H):
            Q, K, V = qs[a:b, h], ks[a:b, h], vs[a:b, h]
            y[a:b, h] = np.tril(Q @ K.T) @ V
            if init is not None:
                y[a:b, h] += Q @ np.asarray(init[s, h], dtype=np.float64)
    return y


def layer(q, k, v, g, w, seg, eps=1e-6, init=None):
    y = attention(q, k, v, seg, init)
    T, H, D = y.shape
    flat = y.reshape(T, H * D)
    rms = np.sqrt(np.mean(flat * flat, axis=1) + eps)
    out = flat / rms[:, None] * np.asarray(w, np.float64)[None, :] * expit(np.asarray(g, np.float64).reshape(T, H * D))
    return out.reshape(T, H, D)
