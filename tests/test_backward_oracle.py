"""Pins of the reverse-pass reference (oracle/backward.py): central finite differences of
the fp64 oracle's loss, and torch autograd through a plain PyTorch statement of the
product form (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
from oracle.backward import backward


def _case(rng, B=1, T=7, Hqk=1, Hv=2, Dk=3, Dv=4, N_lens=None, per_key=False):
    q = rng.standard_normal((B, T, Hqk, Dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, T, Hqk, Dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, Dv))
    beta = rng.uniform(0.1, 1.9, (B, T, Hv))
    g = -rng.uniform(0.0, 0.5, (B, T, Hv, Dk) if per_key else (B, T, Hv))
    return q, k, v, beta, g


def _loss(fwd_out, do, dfin):
    o, fin = fwd_out
    return float(np.sum(o * do) + np.sum(fin * dfin))


@pytest.mark.parametrize("per_key", [False, True])
def test_finite_differences_packed_gqa(per_key):
    """Every input of a packed GQA case, central differences of L = <o, do> + <M_T, dM_T>
    through the oracle of record (dn_oracle.c); one log decay per head, or per key channel."""
    rng = np.random.default_rng(1)
    lens = [4, 0, 5]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, beta, g = _case(rng, T=T, per_key=per_key)
    init = rng.standard_normal((len(lens), 2, 3, 4))
    do = rng.standard_normal(v.shape)
    dfin = rng.standard_normal(init.shape)
    scale = 0.7
    grads = backward(q, k, v, beta, g, init, do, dfin, cu, scale)
    args = dict(q=q, k=k, v=v, beta=beta, g=g, init=init)
    names = dict(q="dq", k="dk", v="dv", beta="dbeta", g="dg", init="dinit")
    eps = 1e-6
    for name, x in args.items():
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap, am = dict(args, **{name: xp}), dict(args, **{name: xm})
            lp = _loss(oracle.recurrent(ap["q"], ap["k"], ap["v"], ap["beta"], ap["g"], ap["init"], cu, scale), do, dfin)
            lm = _loss(oracle.recurrent(am["q"], am["k"], am["v"], am["beta"], am["g"], am["init"], cu, scale), do, dfin)
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grads[names[name]], num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_torch_autograd_of_the_product_form():
    """Autograd through S_t = e^{g_t} S_{t-1} (I - beta k k^T) + beta v k^T, o_t = S_t q_t
    written with torch matrices (fp64), batch rows, no gate and with it."""
    rng = np.random.default_rng(2)
    for gated in (False, True):
        q, k, v, beta, g = _case(rng, B=2, T=6, Hqk=2, Hv=2, Dk=4, Dv=3)
        g = g if gated else None
        do = rng.standard_normal(v.shape)
        tq, tk, tv, tb = (torch.tensor(a, requires_grad=True) for a in (q, k, v, beta))
        tg = torch.tensor(g, requires_grad=True) if gated else None
        loss = 0.0
        for b in range(2):
            for h in range(2):
                S = torch.zeros(3, 4, dtype=torch.float64)
                for t in range(6):
                    kt = tk[b, t, h][:, None]
                    if gated:
                        S = torch.exp(tg[b, t, h]) * S
                    S = S @ (torch.eye(4, dtype=torch.float64) - tb[b, t, h] * (kt @ kt.T)) + tb[b, t, h] * (tv[b, t, h][:, None] @ kt.T)
                    loss = loss + (S @ tq[b, t, h]) @ torch.tensor(do[b, t, h])
        loss.backward()
        grads = backward(q, k, v, beta, g, None, do)
        np.testing.assert_allclose(grads["dq"], tq.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(grads["dk"], tk.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(grads["dv"], tv.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(grads["dbeta"], tb.grad.numpy(), rtol=1e-10, atol=1e-12)
        if gated:
            np.testing.assert_allclose(grads["dg"], tg.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_torch_autograd_of_the_product_form_channel_gates():
    """Autograd through S_t = S_{t-1} diag(e^{g_t}) (I - beta k k^T) + beta v k^T, o_t = S_t
    q_t, with a log decay per key channel (fp64 torch matrices)."""
    rng = np.random.default_rng(3)
    q, k, v, beta, g = _case(rng, B=2, T=6, Hqk=2, Hv=2, Dk=4, Dv=3, per_key=True)
    do = rng.standard_normal(v.shape)
    dfin = rng.standard_normal((2, 2, 4, 3))
    tq, tk, tv, tb, tg = (torch.tensor(a, requires_grad=True) for a in (q, k, v, beta, g))
    loss = 0.0
    for b in range(2):
        for h in range(2):
            S = torch.zeros(3, 4, dtype=torch.float64)
            for t in range(6):
                kt = tk[b, t, h][:, None]
                S = S @ torch.diag(torch.exp(tg[b, t, h]))
                S = S @ (torch.eye(4, dtype=torch.float64) - tb[b, t, h] * (kt @ kt.T)) + tb[b, t, h] * (tv[b, t, h][:, None] @ kt.T)
                loss = loss + (S @ tq[b, t, h]) @ torch.tensor(do[b, t, h])
            loss = loss + torch.sum(S.T * torch.tensor(dfin[b, h]))
    loss.backward()
    grads = backward(q, k, v, beta, g, None, do, dfin)
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv), ("dbeta", tb), ("dg", tg)):
        np.testing.assert_allclose(grads[name], t.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def test_finite_differences_in_call_normalisation():
    """Raw q and k normalised inside the rule: central differences of the loss through the C
    oracle with qk_l2norm, for q and k (the other inputs see the normalised vectors only)."""
    rng = np.random.default_rng(4)
    q, k, v, beta, g = _case(rng, T=6, Hqk=1, Hv=2, Dk=3, Dv=4)
    q = q * rng.uniform(0.5, 3.0, q.shape[:-1] + (1,))
    k = k * rng.uniform(0.5, 3.0, k.shape[:-1] + (1,))
    init = rng.standard_normal((1, 2, 3, 4))
    do = rng.standard_normal(v.shape)
    dfin = rng.standard_normal(init.shape)
    eps = 1e-3
    grads = backward(q, k, v, beta, g, init, do, dfin, None, 0.9, qk_l2norm=True, eps=eps)
    h = 1e-6
    for name, x in (("q", q), ("k", k)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            qp, kp = (xp, k) if name == "q" else (q, xp)
            qm, km = (xm, k) if name == "q" else (q, xm)
            lp = _loss(oracle.recurrent(qp, kp, v, beta, g, init, None, 0.9, qk_l2norm=True, eps=eps), do, dfin)
            lm = _loss(oracle.recurrent(qm, km, v, beta, g, init, None, 0.9, qk_l2norm=True, eps=eps), do, dfin)
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grads["d" + name], num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_torch_autograd_through_the_normalisation():
    """Autograd of the product form with q, k replaced by x / sqrt(|x|^2 + eps) (fp64)."""
    rng = np.random.default_rng(5)
    q, k, v, beta, g = _case(rng, B=1, T=5, Hqk=1, Hv=1, Dk=4, Dv=3)
    q, k = q * 2.5, k * 0.4
    eps = 1e-2
    do = rng.standard_normal(v.shape)
    tq, tk = torch.tensor(q, requires_grad=True), torch.tensor(k, requires_grad=True)
    nrm = lambda x: x / torch.sqrt(torch.sum(x * x, dim=-1, keepdim=True) + eps)
    qh, kh = nrm(tq), nrm(tk)
    S = torch.zeros(3, 4, dtype=torch.float64)
    loss = 0.0
    for t in range(5):
        kt = kh[0, t, 0][:, None]
        S = float(np.exp(g[0, t, 0])) * S
        S = S @ (torch.eye(4, dtype=torch.float64) - beta[0, t, 0] * (kt @ kt.T)) + beta[0, t, 0] * (torch.tensor(v[0, t, 0])[:, None] @ kt.T)
        loss = loss + (S @ qh[0, t, 0]) @ torch.tensor(do[0, t, 0])
    loss.backward()
    grads = backward(q, k, v, beta, g, None, do, qk_l2norm=True, eps=eps)
    np.testing.assert_allclose(grads["dq"], tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(grads["dk"], tk.grad.numpy(), rtol=1e-10, atol=1e-12)
