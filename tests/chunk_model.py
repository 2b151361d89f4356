"""fp64 model of the chunkwise (WY/UT) form of the gated delta rule, test-only.

This is the algebra the HIP prefill kernels implement, written plainly in numpy so
that it can be checked against the token-by-token oracle before (and independently
of) any GPU code.  It shares no code with the HIP library and does not import the
oracle.

Derivation (from the update of the frankenstein DeltaNet page's module docstring,
with the gate order of the nnterp LinearAttention class text).  Inside one chunk of
n tokens starting from the key-major state M0 = S0^T, with gamma_r = sum_{i<=r} g_i:

  S_r = exp(gamma_r) S0 + sum_{i<=r} exp(gamma_r - gamma_i) delta_i k_i^T,
  delta_r = beta_r (v_r - exp(g_r) S_{r-1} k_r).

Substituting the first line into the second gives, with Delta = [delta_r^T]_r,

  (I + A) Delta = R,   A_ri = beta_r exp(gamma_r - gamma_i) k_r.k_i  (i < r),
  R = diag(beta) (V - diag(exp(gamma)) K M0).

So Delta = T R with T = (I + A)^{-1} (unit lower triangular), and

  O     = scale * (diag(exp(gamma)) Q M0 + P Delta),  P_ri = exp(gamma_r - gamma_i) q_r.k_i (i <= r)
  M_new = exp(gamma_{n-1}) M0 + Ktil^T Delta,           Ktil_i = exp(gamma_{n-1} - gamma_i) k_i.

``quant`` (optional) rounds the operands the GPU feeds to its bf16 matrix cores, so
the model also predicts the bf16 path's error.
"""
from __future__ import annotations

import numpy as np


def blocked_unit_lower_inverse(A: np.ndarray, bs: int = 16) -> np.ndarray:
    """(I + A)^{-1} for strictly lower-triangular A, by bs x bs blocks: forward
    substitution inside each diagonal block, then the off-diagonal blocks diagonal
    by diagonal, T_ij = -T_ii sum_{j<=m<i} A_im T_mj."""
    n = A.shape[0]
    nb = (n + bs - 1) // bs
    T = np.zeros_like(A)
    for b in range(nb):
        s, e = b * bs, min(n, (b + 1) * bs)
        for r in range(s, e):
            T[r, s:e] = 0.0
            T[r, r] = 1.0
            for m in range(s, r):
                T[r, s:e] -= A[r, m] * T[m, s:e]
    for d in range(1, nb):
        for i in range(d, nb):
            j = i - d
            si, ei = i * bs, min(n, (i + 1) * bs)
            sj, ej = j * bs, min(n, (j + 1) * bs)
            X = np.zeros((ei - si, ej - sj))
            for m in range(j, i):
                sm, em = m * bs, min(n, (m + 1) * bs)
                X += A[si:ei, sm:em] @ T[sm:em, sj:ej]
            T[si:ei, sj:ej] = -T[si:ei, si:ei] @ X
    return T


def chunked(q, k, v, beta, g=None, init=None, cu_seqlens=None, scale=1.0, C=64,
            quant=None, blocked=True):
    """Same signature and result as the oracle, computed chunk by chunk."""
    Q = (lambda x: x) if quant is None else quant
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    r = Hv // Hqk
    qf, kf, vf = q.reshape(B * T, Hqk, Dk), k.reshape(B * T, Hqk, Dk), v.reshape(B * T, Hv, Dv)
    bf = beta.reshape(B * T, Hv)
    gf = None if g is None else g.reshape(B * T, Hv)
    cu = (np.arange(B + 1) * T) if cu_seqlens is None else np.asarray(cu_seqlens)
    N = len(cu) - 1
    o = np.zeros((B * T, Hv, Dv))
    final = np.zeros((N, Hv, Dk, Dv))
    for n in range(N):
        for h in range(Hv):
            hq = h // r
            M = np.zeros((Dk, Dv)) if init is None else np.array(init[n, h], dtype=np.float64)
            for s in range(cu[n], cu[n + 1], C):
                e = min(s + C, cu[n + 1])
                K, Qc, V, bt = kf[s:e, hq], qf[s:e, hq], vf[s:e, h], bf[s:e, h]
                gam = np.zeros(e - s) if gf is None else np.cumsum(gf[s:e, h])
                diff = gam[:, None] - gam[None, :]
                low = np.tril(np.ones((e - s, e - s), dtype=bool))
                D = np.where(low, np.exp(np.where(low, diff, 0.0)), 0.0)
                A = np.tril(bt[:, None] * D * (K @ K.T), -1)
                Tm = blocked_unit_lower_inverse(A) if blocked else np.linalg.inv(np.eye(e - s) + A)
                Mq = Q(M)
                R = bt[:, None] * (V - np.exp(gam)[:, None] * (K @ Mq))
                Delta = Q(Tm) @ Q(R)
                P = D * (Qc @ K.T)
                o[s:e, h] = scale * (np.exp(gam)[:, None] * (Qc @ Mq) + Q(P) @ Q(Delta))
                tail = np.exp(gam[-1] - gam)
                M = np.exp(gam[-1]) * M + K.T @ Q(tail[:, None] * Delta)
            final[n, h] = M
    return o.reshape(B, T, Hv, Dv), final
