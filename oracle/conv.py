"""fp64 reference of the short causal convolution in front of the rule -- TEST
INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): only the tests, the smoke check and the
benchmark's CPU leg may import it, and the HIP library never calls it.

The mutichung "DeltaNet" page's block flowchart puts, on each of the q/k and v branches,
a "Conv" box then a "SiLU" box between the projection and the rule (then the L2 norm on
q and k), and calls the convolutions depthwise-separable, generalising the shift SSM.
Reading: per channel c a causal filter of width W (weights w[c, 0..W-1], the last tap on
the current token, an optional bias), then silu:

    y_t[c] = silu(b[c] + sum_{j<W} w[c, j] x_{t-W+1+j}[c])

Inputs before a sequence's first token come from its conv state -- the W - 1 inputs before
it, oldest first, ``[N, C, W - 1]`` -- or are zero.  The state after a sequence is its
last W - 1 inputs (taking state entries when the sequence is shorter than W - 1).  A
decode step is the same with T = 1, the state shifted by one.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

__all__ = ["causal_conv", "conv_qkv"]


def causal_conv(x: np.ndarray, weight: np.ndarray, bias: Optional[np.ndarray] = None,
                cu_seqlens: Optional[np.ndarray] = None, init_state: Optional[np.ndarray] = None,
                activation: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """x ``[B, T, C]`` (B == 1 with ``cu_seqlens`` ``[N + 1]``), weight ``[C, W]``, bias
    ``[C]``, init_state ``[N, C, W - 1]`` -> (y ``[B, T, C]``, final state ``[N, C, W - 1]``),
    fp64."""
    x = np.asarray(x, dtype=np.float64)
    B, T, C = x.shape
    w = np.asarray(weight, dtype=np.float64)
    W = w.shape[1]
    if cu_seqlens is None:
        cu = np.arange(B + 1) * T
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        if B != 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
            raise ValueError("packed sequences need B == 1 and offsets from 0 to T")
    N = len(cu) - 1
    flat = x.reshape(B * T, C)
    y = np.zeros_like(flat)
    final = np.zeros((N, C, W - 1))
    for n in range(N):
        prev = np.zeros((W - 1, C)) if init_state is None else np.asarray(init_state[n], dtype=np.float64).T
        seq = np.concatenate([prev, flat[cu[n]:cu[n + 1]]], axis=0)   # [W - 1 + L, C]
        for t in range(cu[n + 1] - cu[n]):
            acc = np.zeros(C) if bias is None else np.asarray(bias, dtype=np.float64).copy()
            for j in range(W):
                acc = acc + w[:, j] * seq[t + j]
            y[cu[n] + t] = acc / (1.0 + np.exp(-acc)) if activation else acc
        final[n] = seq[len(seq) - (W - 1):].T
    return y.reshape(B, T, C), final


def conv_qkv(x: np.ndarray, weight: np.ndarray, bias: Optional[np.ndarray], Hqk: int, Hv: int,
             Dk: int, Dv: int, cu_seqlens: Optional[np.ndarray] = None,
             init_state: Optional[np.ndarray] = None, activation: bool = True,
             qk_l2norm: bool = True, eps: float = 1e-6):
    """The prologue of the same flowchart in one function: the convolution above over
    x = [q | k | v] channels ``[B, T, 2 Hqk Dk + Hv Dv]``, its output split into q, k
    ``[B, T, Hqk, Dk]`` and v ``[B, T, Hv, Dv]``, then (the flowchart's "L2 Norm" box on the
    q and k branches) every q and k head replaced by u / sqrt(|u|^2 + eps).  Returns
    (q, k, v, final state), fp64."""
    y, final = causal_conv(x, weight, bias, cu_seqlens, init_state, activation)
    B, T, C = y.shape
    if C != 2 * Hqk * Dk + Hv * Dv:
        raise ValueError("x must hold 2 Hqk Dk + Hv Dv channels")
    q = y[..., :Hqk * Dk].reshape(B, T, Hqk, Dk)
    k = y[..., Hqk * Dk:2 * Hqk * Dk].reshape(B, T, Hqk, Dk)
    v = y[..., 2 * Hqk * Dk:].reshape(B, T, Hv, Dv)
    if qk_l2norm:
        q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)
        k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    return q, k, v, final
