"""fp64 reverse pass of the gated delta rule, token by token -- TEST INFRASTRUCTURE ONLY
(see ``oracle/__init__.py``): only the tests, the smoke check and the benchmark's CPU leg
may import it, and the HIP library never calls it.

The forward rule is the one ``dn_oracle.c`` runs (frankenstein "DeltaNet Attention" page,
update equation; gate first per the nnterp "linear_attention" class text; read after the
write), per (sequence, value head), with the state stored key-major, M = S^T [Dk, Dv]:

    M'_t = a_t M_{t-1},  a_t = exp(g_t)
    r_t  = M'_t^T k_t,   delta_t = beta_t (v_t - r_t)
    M_t  = M'_t + k_t delta_t^T,      o_t = scale M_t^T q_t

Given dL/do_t and dL/dM_T, the reverse pass walks the tokens backwards with the adjoint
G = dL/dM_t (chain rule on each line above):

    G    += scale q_t do_t^T,          dq_t = scale M_t do_t
    dd    = G^T k_t                    (dL/d delta_t)
    dv_t  = beta_t dd,                 dbeta_t = dd . (v_t - r_t)
    dk_t  = G delta_t - beta_t M'_t dd
    G'    = G - beta_t k_t dd^T        (dL/dM'_t)
    dg_t  = <G', M'_t>,                G <- a_t G'   (dL/dM_{t-1})

and dL/dM_0 is G after the first token.  With a log decay per key channel (the nnterp
page's ChannelGates), a_t is a vector over the rows of M: M'_t = diag(a_t) M_{t-1}, and
the same chain rule gives dg_t[i] = sum_j G'[i, j] M'_t[i, j] and G <- diag(a_t) G'.  Value head h reads query/key head h / (Hv/Hqk):
dq and dk are summed over the value heads that share a query/key head.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

__all__ = ["backward"]


def _unnormalise(x, dxh, eps):
    """dL/dx from dL/dx_hat for x_hat = x / n, n = sqrt(|x|^2 + eps) over the last axis:
    dx = (dx_hat - x (x . dx_hat) / n^2) / n, and 0 where n = 0 (the rule's zero vector)."""
    n2 = np.sum(x * x, axis=-1, keepdims=True) + eps
    n = np.sqrt(n2)
    safe = np.where(n2 > 0, n2, 1.0)
    out = (dxh - x * np.sum(x * dxh, axis=-1, keepdims=True) / safe) / np.sqrt(safe)
    return np.where(n > 0, out, 0.0)


def backward(q, k, v, beta, g, init, do, dfinal=None, cu_seqlens=None, scale: float = 1.0,
             qk_l2norm: bool = False, eps: float = 1e-6):
    """Gradients of the rule.  Shapes as ``oracle.recurrent`` (q, k ``[B, T, Hqk, Dk]``, v
    ``[B, T, Hv, Dv]``, beta ``[B, T, Hv]``, g ``[B, T, Hv]``, ``[B, T, Hv, Dk]`` (a log
    decay per key channel) or None, init ``[N, Hv, Dk, Dv]`` or None), do ``[B, T, Hv, Dv]``,
    dfinal ``[N, Hv, Dk, Dv]`` or None.  Returns a dict of fp64 arrays dq, dk, dv, dbeta,
    dg (g's shape; None without g), dinit.

    With ``qk_l2norm`` the rule reads q / sqrt(|q|^2 + eps) and k / sqrt(|k|^2 + eps) (the
    in-call normalisation of ``oracle.recurrent``): the pass runs on the normalised vectors
    and dq, dk are taken back through the normalisation."""
    if qk_l2norm:
        q, k = np.asarray(q, dtype=np.float64), np.asarray(k, dtype=np.float64)
        nq = np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)
        nk = np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
        qh = np.where(nq > 0, q / np.where(nq > 0, nq, 1.0), 0.0)
        kh = np.where(nk > 0, k / np.where(nk > 0, nk, 1.0), 0.0)
        out = backward(qh, kh, v, beta, g, init, do, dfinal, cu_seqlens, scale)
        out["dq"] = _unnormalise(q, out["dq"], eps)
        out["dk"] = _unnormalise(k, out["dk"], eps)
        return out
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    beta, do = np.asarray(beta, dtype=np.float64), np.asarray(do, dtype=np.float64)
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    grp = Hv // Hqk
    cu = np.arange(B + 1) * T if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    fl = lambda a, *tail: a.reshape((B * T,) + tail)
    qf, kf, vf = fl(q, Hqk, Dk), fl(k, Hqk, Dk), fl(v, Hv, Dv)
    bf, df = fl(beta, Hv), fl(do, Hv, Dv)
    per_key = g is not None and np.ndim(g) == 4
    gshape = None if g is None else np.shape(g)
    gf = None if g is None else (fl(np.asarray(g, dtype=np.float64), Hv, Dk) if per_key
                                 else fl(np.asarray(g, dtype=np.float64), Hv))
    rows = (lambda a: a[:, None]) if per_key else (lambda a: a)   # decay of each row of M
    dq, dk = np.zeros_like(qf), np.zeros_like(kf)
    dv, dbeta = np.zeros_like(vf), np.zeros_like(bf)
    dg = None if g is None else np.zeros_like(gf)
    dinit = np.zeros((N, Hv, Dk, Dv))
    for n in range(N):
        for h in range(Hv):
            hq = h // grp
            M = np.zeros((Dk, Dv)) if init is None else np.array(init[n, h], dtype=np.float64)
            Ms, Mp = [], []                     # M_t and M'_t of each token (forward)
            for t in range(cu[n], cu[n + 1]):
                a = 1.0 if gf is None else rows(np.exp(gf[t, h]))
                Mpt = a * M
                r = Mpt.T @ kf[t, hq]
                M = Mpt + np.outer(kf[t, hq], bf[t, h] * (vf[t, h] - r))
                Mp.append(Mpt)
                Ms.append(M)
            G = np.zeros((Dk, Dv)) if dfinal is None else np.array(dfinal[n, h], dtype=np.float64)
            for i, t in reversed(list(enumerate(range(cu[n], cu[n + 1])))):
                kt, qt = kf[t, hq], qf[t, hq]
                Mpt, Mt = Mp[i], Ms[i]
                r = Mpt.T @ kt
                delta = bf[t, h] * (vf[t, h] - r)
                G = G + scale * np.outer(qt, df[t, h])
                dq[t, hq] += scale * (Mt @ df[t, h])
                dd = G.T @ kt
                dv[t, h] = bf[t, h] * dd
                dbeta[t, h] = dd @ (vf[t, h] - r)
                dk[t, hq] += G @ delta - bf[t, h] * (Mpt @ dd)
                Gp = G - bf[t, h] * np.outer(kt, dd)
                a = 1.0 if gf is None else rows(np.exp(gf[t, h]))
                if dg is not None:
                    dg[t, h] = np.sum(Gp * Mpt, axis=1) if per_key else np.sum(Gp * Mpt)
                G = a * Gp
            dinit[n, h] = G
    out = dict(dq=dq.reshape(q.shape), dk=dk.reshape(k.shape), dv=dv.reshape(v.shape),
               dbeta=dbeta.reshape(beta.shape), dg=None if dg is None else dg.reshape(gshape),
               dinit=dinit)
    return out
