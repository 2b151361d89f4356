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


def chunked_backward(q, k, v, beta, g, init, do, dfinal=None, cu_seqlens=None, scale=1.0, C=64):
    """Reverse pass of the chunked form, chunk by chunk from the chunk-start states (the
    algebra the HIP chunkwise reverse pass implements).  Per chunk, with dM' the gradient
    of the state after it and dO of its outputs:

      dDelta = scale P^T dO + diag(tail) K dM'        dR = T^T dDelta
      dV = diag(beta) dR                               dX = -diag(beta exp(gamma)) dR
      dM = exp(gamma_L) dM' + scale Q^T diag(exp(gamma)) dO + K^T dX
      dA = -(dR Delta^T) strictly lower,   dP = scale (dO Delta^T) lower with the diagonal
      dQ = scale diag(exp(gamma)) dO M^T + (dP o D) K
      dK = dX M^T + diag(tail) Delta dM'^T + (W + W^T) K + (dP o D)^T Q,  W = dA o diag(beta) D
      dbeta_r = (V - diag(exp(gamma)) X)_r . dR_r + sum_i dA_ri D_ri k_r.k_i
      dgamma_r = scale exp(gamma_r) (Q M)_r . dO_r - beta_r exp(gamma_r) X_r . dR_r
                 + rowsum_r(dA o A) - colsum_r(dA o A) + rowsum_r(dP o P) - colsum_r(dP o P) - c_r
                 (+ exp(gamma_L) <M, dM'> + sum_r c_r on the chunk's last row),
      c_r = tail_r (K dM')_r . Delta_r,   dg_i = sum_{r >= i in the chunk} dgamma_r.

    Returns the dict of ``oracle.backward.backward``."""
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    grp = Hv // Hqk
    qf, kf, vf = q.reshape(B * T, Hqk, Dk), k.reshape(B * T, Hqk, Dk), v.reshape(B * T, Hv, Dv)
    bf = beta.reshape(B * T, Hv)
    dof = do.reshape(B * T, Hv, Dv)
    gf = None if g is None else g.reshape(B * T, Hv)
    cu = (np.arange(B + 1) * T) if cu_seqlens is None else np.asarray(cu_seqlens)
    N = len(cu) - 1
    dq, dk = np.zeros_like(qf, dtype=np.float64), np.zeros_like(kf, dtype=np.float64)
    dv, dbeta = np.zeros_like(vf, dtype=np.float64), np.zeros_like(bf, dtype=np.float64)
    dg = None if g is None else np.zeros_like(gf, dtype=np.float64)
    dinit = np.zeros((N, Hv, Dk, Dv))
    for n in range(N):
        for h in range(Hv):
            hq = h // grp
            starts = list(range(cu[n], cu[n + 1], C))
            # forward sweep: the state at each chunk start
            M = np.zeros((Dk, Dv)) if init is None else np.array(init[n, h], dtype=np.float64)
            Ms = []
            for s in starts:
                e = min(s + C, cu[n + 1])
                K, V, bt = kf[s:e, hq], vf[s:e, h], bf[s:e, h]
                gam = np.zeros(e - s) if gf is None else np.cumsum(gf[s:e, h])
                low = np.tril(np.ones((e - s, e - s), dtype=bool))
                D = np.where(low, np.exp(np.where(low, gam[:, None] - gam[None, :], 0.0)), 0.0)
                A = np.tril(bt[:, None] * D * (K @ K.T), -1)
                Delta = np.linalg.solve(np.eye(e - s) + A, bt[:, None] * (V - np.exp(gam)[:, None] * (K @ M)))
                Ms.append(M)
                M = np.exp(gam[-1]) * M + K.T @ (np.exp(gam[-1] - gam)[:, None] * Delta)
            dMp = np.zeros((Dk, Dv)) if dfinal is None else np.array(dfinal[n, h], dtype=np.float64)
            for s, M in reversed(list(zip(starts, Ms))):
                e = min(s + C, cu[n + 1])
                L = e - s
                K, Qc, V, bt, dO = kf[s:e, hq], qf[s:e, hq], vf[s:e, h], bf[s:e, h], dof[s:e, h]
                gam = np.zeros(L) if gf is None else np.cumsum(gf[s:e, h])
                eg, tail = np.exp(gam), np.exp(gam[-1] - gam)
                low = np.tril(np.ones((L, L), dtype=bool))
                D = np.where(low, np.exp(np.where(low, gam[:, None] - gam[None, :], 0.0)), 0.0)
                Gk = D * (K @ K.T)
                A = np.tril(bt[:, None] * Gk, -1)
                Tm = np.linalg.inv(np.eye(L) + A)
                P = D * (Qc @ K.T)
                X = K @ M
                Rt = V - eg[:, None] * X
                Delta = Tm @ (bt[:, None] * Rt)
                KdM = K @ dMp
                dDelta = scale * P.T @ dO + tail[:, None] * KdM
                dR = Tm.T @ dDelta
                dv[s:e, h] = bt[:, None] * dR
                dX = -(bt * eg)[:, None] * dR
                dA = np.tril(-(dR @ Delta.T), -1)
                dP = np.tril(scale * (dO @ Delta.T))
                W = dA * bt[:, None] * D
                Z = dP * D
                dq[s:e, hq] += scale * eg[:, None] * (dO @ M.T) + Z @ K
                dk[s:e, hq] += dX @ M.T + tail[:, None] * (Delta @ dMp.T) + (W + W.T) @ K + Z.T @ Qc
                dbeta[s:e, h] = np.sum(Rt * dR, axis=1) + np.sum(dA * Gk, axis=1)
                if dg is not None:
                    c = tail * np.sum(KdM * Delta, axis=1)
                    dA_A, dP_P = dA * A, dP * P
                    dgam = (scale * eg * np.sum((Qc @ M) * dO, axis=1) - bt * eg * np.sum(X * dR, axis=1)
                            + dA_A.sum(1) - dA_A.sum(0) + dP_P.sum(1) - dP_P.sum(0) - c)
                    dgam[-1] += np.exp(gam[-1]) * np.sum(M * dMp) + c.sum()
                    dg[s:e, h] = np.cumsum(dgam[::-1])[::-1]
                dMp = np.exp(gam[-1]) * dMp + scale * Qc.T @ (eg[:, None] * dO) + K.T @ dX
            dinit[n, h] = dMp
    return dict(dq=dq.reshape(q.shape), dk=dk.reshape(k.shape), dv=dv.reshape(v.shape),
                dbeta=dbeta.reshape(beta.shape), dg=None if dg is None else dg.reshape(g.shape),
                dinit=dinit)
