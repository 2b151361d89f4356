"""Tiny-input fp64 twins of the delta rule, one per reading the pages give.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Each function runs one
sequence of one head with pure-Python loops over tokens and explicit matrices.  They
are written from different statements of the same update than ``dn_oracle.c`` is,
so agreement between them pins the oracle.

S is the pages' value-by-key state (``S k = v``), shape ``[Dv, Dk]``.  Every
function takes q, k ``[T, Dk]``, v ``[T, Dv]``, beta ``[T]``, g ``[T]`` (or ``[T, Dk]``, per
key channel, for :func:`product_form`) or None,
S0 ``[Dv, Dk]`` or None, and returns ``(o [T, Dv], S_T [Dv, Dk])``.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

__all__ = ["product_form", "retrieve_interpolate_form", "per_token_states"]


def _start(k, v, S0):
    Dk, Dv = k.shape[1], v.shape[1]
    return np.zeros((Dv, Dk)) if S0 is None else np.array(S0, dtype=np.float64)


def product_form(q, k, v, beta, g=None, S0=None, scale: float = 1.0
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """Frankenstein "DeltaNet Attention" page, module docstring (update equation):
    ``S_t = S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T``, written with the
    explicit d_k x d_k matrix ``I - beta k k^T``.  The gate of the nnterp
    LinearAttention class text multiplies the previous state by ``exp(g_t)`` before
    the update; the read is ``o_t = scale * S_t q_t``.
    """
    S = _start(k, v, S0)
    T, Dk = k.shape
    I = np.eye(Dk)
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        kt = k[t][:, None]
        S = _decayed(S, g, t) @ (I - beta[t] * (kt @ kt.T)) + beta[t] * (v[t][:, None] @ kt.T)
        o[t] = scale * (S @ q[t])
    return o, S


def _decayed(S, g, t):
    """The state after token t's gate: exp(g_t) S for one gate per head, or
    S diag(exp(g_t)) for a gate per key channel (g[t] a vector of length Dk; the nnterp
    page's ChannelGates, read as the key channels of S keeping exp(g_t[i]) each)."""
    if g is None:
        return S
    a = np.exp(np.asarray(g[t], dtype=np.float64))
    if a.ndim == 0:
        return a * S
    return S @ np.diag(a)


def retrieve_interpolate_form(q, k, v, beta, g=None, S0=None, scale: float = 1.0
                              ) -> Tuple[np.ndarray, np.ndarray]:
    """Mutichung garden "DeltaNet" page, section "The Delta Rule", key-value
    retrieval reading: retrieve ``v_old = S_{t-1} k_t``, blend
    ``v_new = beta v_t + (1 - beta) v_old``, then remove ``v_old k^T`` and write
    ``v_new k^T``.  (On that page the blend and the state equation are run together
    into one display; they are two equations.)  Gate and read as in
    :func:`product_form`.
    """
    S = _start(k, v, S0)
    T = k.shape[0]
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        if g is not None:
            S = np.exp(g[t]) * S
        v_old = S @ k[t]
        v_new = beta[t] * v[t] + (1.0 - beta[t]) * v_old
        S = S - np.outer(v_old, k[t]) + np.outer(v_new, k[t])
        o[t] = scale * (S @ q[t])
    return o, S


def per_token_states(k, v, beta, g=None, S0=None) -> np.ndarray:
    """States ``S_1 .. S_T`` ``[T, Dv, Dk]`` of :func:`product_form` (for invariants
    that hold at every token)."""
    S = _start(k, v, S0)
    T, Dk = k.shape
    I = np.eye(Dk)
    out = np.zeros((T,) + S.shape)
    for t in range(T):
        a = 1.0 if g is None else np.exp(g[t])
        kt = k[t][:, None]
        S = (a * S) @ (I - beta[t] * (kt @ kt.T)) + beta[t] * (v[t][:, None] @ kt.T)
        out[t] = S
    return out
