"""fp64 oracle of the KDA layer's prologue (test infrastructure only).

For each of the q, k, v projections: a causal depthwise convolution of
kernel 4 per channel, whose weight has the checkpoint's shape [H*d, 1, 4]
(Kimi K3 artifact audit, §4.1), an optional SiLU, and for q and k an L2
normalisation over the d channels of every (token, head).  The pages give
the weight shapes and the kernel size only; the activation and the norm's
eps are arguments.  Sequences are packed by cu_seqlens; the conv state of a
sequence is its last 3 inputs per channel, oldest first.

Written from the definition, one sequence at a time, with nothing fused.
Pinned in tests/test_oracle_pins.py (impulse response, numpy.convolve,
unit norm, SiLU closed forms, split-with-state = one shot).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .api import f64

K = 4  # kernel size


def silu(y: np.ndarray) -> np.ndarray:
    return y / (1.0 + np.exp(-y))


def causal_conv(x: np.ndarray, w: np.ndarray, prev: np.ndarray) -> np.ndarray:
    """x [L, C], w [C, 4], prev [3, C] (inputs before x, oldest first) ->
    y[t, c] = sum_i w[c, i] * x[t - 3 + i, c]."""
    xs = np.concatenate([prev, x], axis=0)          # xs[t + 3] = x[t]
    L = x.shape[0]
    y = np.zeros_like(x)
    for i in range(K):
        y += w[:, i][None, :] * xs[i:i + L]
    return y


def l2norm(y: np.ndarray, H: int, d: int, eps: float) -> np.ndarray:
    """y [L, H*d] -> each (token, head) row divided by sqrt(sum of squares + eps)."""
    r = y.reshape(y.shape[0], H, d)
    r = r / np.sqrt(np.sum(r * r, axis=2, keepdims=True) + eps)
    return r.reshape(y.shape)


def shortconv_l2norm(xq, xk, xv, wq, wk, wv, cu_seqlens, H: int, d: int = 128,
                     activation: Optional[str] = "silu", eps: float = 1e-6,
                     state: Optional[np.ndarray] = None
                     ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """xq/xk/xv [T, H, d]; wq/wk/wv [H*d, 4] (or [H*d, 1, 4]); state [N, 3, 3, H*d]
    or None (zeros).  Returns yq, yk, yv [T, H, d] and the state after."""
    xs = [f64(a).reshape(-1, H * d) for a in (xq, xk, xv)]
    ws = [f64(a).reshape(H * d, K) for a in (wq, wk, wv)]
    cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
    N = cu.shape[0] - 1
    st_in = np.zeros((N, 3, K - 1, H * d)) if state is None else f64(state).reshape(N, 3, K - 1, H * d)
    st_out = np.zeros_like(st_in)
    ys = [np.zeros_like(a) for a in xs]
    for n in range(N):
        b, e = int(cu[n]), int(cu[n + 1])
        for z in range(3):
            x = xs[z][b:e]
            y = causal_conv(x, ws[z], st_in[n, z])
            if activation == "silu":
                y = silu(y)
            elif activation is not None:
                raise ValueError("activation must be 'silu' or None")
            if z < 2:
                y = l2norm(y, H, d, eps)
            ys[z][b:e] = y
            st_out[n, z] = np.concatenate([st_in[n, z], x], axis=0)[-(K - 1):]
    T = xs[0].shape[0]
    return (ys[0].reshape(T, H, d), ys[1].reshape(T, H, d), ys[2].reshape(T, H, d), st_out)
