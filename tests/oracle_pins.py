"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every ``pin_*`` function takes ``run`` (a callable with the signature of
``oracle.recurrent``) and raises AssertionError when ``run`` disagrees with the pin.
``test_oracle_pins.py`` applies them to the oracle; ``test_oracle_mutants.py``
applies them to copies of the oracle with planted mistakes and requires that some
pin fails for each copy.

Pages: [P1] frankenstein "DeltaNet Attention" (module docstring, update equation;
forward: q and k L2-normalised, read o_t = S_t q_t); [P2] mutichung garden
"DeltaNet" (section "The Delta Rule": error-correction form, SGD reading,
retrieve/interpolate reading); [P3] nnterp "linear_attention" (LinearAttention:
decay, then write, then read; decays = log of the fraction kept, non-positive;
betas in (0, 1) or (0, 2); state_input None on a fresh prompt).
"""
from __future__ import annotations

import numpy as np

from oracle import brute
from tests.golden import load_hand_worked


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _one(run, q, k, v, beta, g=None, M0=None, scale=1.0):
    """One sequence, one head: 2-D inputs -> (o [T, Dv], M_T [Dk, Dv])."""
    T, Dk = k.shape
    Dv = v.shape[1]
    o, fin = run(q.reshape(1, T, 1, Dk), k.reshape(1, T, 1, Dk), v.reshape(1, T, 1, Dv),
                 beta.reshape(1, T, 1), None if g is None else g.reshape(1, T, 1),
                 None if M0 is None else M0.reshape(1, 1, Dk, Dv), scale=scale)
    return o.reshape(T, Dv), fin.reshape(Dk, Dv)


def _rand_seq(rng, T, Dk, Dv, gated=True, init=True, beta_hi=1.0):
    q = _unit(rng.standard_normal((T, Dk)))
    k = _unit(rng.standard_normal((T, Dk)))
    v = rng.standard_normal((T, Dv))
    beta = beta_hi * rng.uniform(0.05, 1.0, T)
    g = -0.3 * rng.uniform(0, 1, T) if gated else None
    M0 = 0.5 * rng.standard_normal((Dk, Dv)) if init else None
    return q, k, v, beta, g, M0


def _close(a, b, tol, what):
    a, b = np.asarray(a), np.asarray(b)
    if a.shape != b.shape:
        raise AssertionError(f"{what}: shape {a.shape} != {b.shape}")
    err = np.max(np.abs(a - b)) / max(1.0, np.max(np.abs(b)))
    if not err <= tol:
        raise AssertionError(f"{what}: max rel error {err:.3e} > {tol:.1e}")


# --------------------------------------------------------------------------- pins

def pin_hand_worked(run):
    """tests/golden/hand_worked.txt: three examples worked by hand ([P1] update
    equation with [P3] gate order), including a reflection (beta = 2) and d_k != d_v."""
    for name, c in load_hand_worked().items():
        o, fin = _one(run, c["q"], c["k"], c["v"], c["beta"], c["g"], c["init"])
        _close(o, c["o"], 1e-13, f"{name} o")
        _close(fin, c["final"], 1e-13, f"{name} final")


def pin_product_form(run):
    """[P1] product form S(I - beta k k^T) + beta v k^T, with explicit matrices, equals
    the oracle (which codes [P2]'s error-correction form)."""
    rng = np.random.default_rng(11)
    for (T, Dk, Dv, gated, init, bh) in [(9, 4, 4, False, False, 1.0), (23, 5, 7, True, True, 1.0),
                                        (17, 8, 3, True, True, 2.0), (40, 16, 16, True, False, 1.0)]:
        q, k, v, beta, g, M0 = _rand_seq(rng, T, Dk, Dv, gated, init, bh)
        o, fin = _one(run, q, k, v, beta, g, M0, scale=0.7)
        ob, Sb = brute.product_form(q, k, v, beta, g, None if M0 is None else M0.T, scale=0.7)
        _close(o, ob, 1e-12, "o vs product form")
        _close(fin, Sb.T, 1e-12, "state vs product form")


def pin_retrieve_interpolate(run):
    """[P2] key-value retrieval reading (v_old, v_new = beta v + (1 - beta) v_old,
    remove v_old k^T, write v_new k^T) gives the oracle's states and outputs."""
    rng = np.random.default_rng(12)
    q, k, v, beta, g, M0 = _rand_seq(rng, 31, 6, 5, True, True, 2.0)
    o, fin = _one(run, q, k, v, beta, g, M0)
    ob, Sb = brute.retrieve_interpolate_form(q, k, v, beta, g, M0.T)
    _close(o, ob, 1e-12, "o vs retrieve/interpolate")
    _close(fin, Sb.T, 1e-12, "state vs retrieve/interpolate")


def pin_beta_zero(run):
    """beta = 0 writes nothing: the plain rule leaves S unchanged (o_t = S_0 q_t); the
    gated rule only decays it, S_t = exp(sum_{u<=t} g_u) S_0."""
    rng = np.random.default_rng(13)
    q, k, v, _, g, M0 = _rand_seq(rng, 12, 6, 4, True, True)
    beta = np.zeros(12)
    o, fin = _one(run, q, k, v, beta, None, M0)
    _close(fin, M0, 0, "beta=0 plain state")
    _close(o, q @ M0, 1e-14, "beta=0 plain output")
    o, fin = _one(run, q, k, v, beta, g, M0)
    gam = np.cumsum(g)
    _close(fin, np.exp(gam[-1]) * M0, 1e-13, "beta=0 decay-only state")
    _close(o, np.exp(gam)[:, None] * (q @ M0), 1e-13, "beta=0 decay-only output")


def pin_exact_recall(run):
    """beta = 1 with orthonormal keys recalls exactly: S k_s = v_s, so the key-major
    state is K^T V ([P1]: the rule removes the old association before writing; the
    docstring's perfect-recall claim at kernel level).  With a gate, pair s has
    decayed by exp(sum_{u>s} g_u) by the end; reads o_t = sum_{s<=t} (k_s . q_t) v_s."""
    rng = np.random.default_rng(14)
    Dk, Dv, T = 16, 24, 16
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    k = Qm.T[:T]                               # orthonormal rows
    v = rng.standard_normal((T, Dv))
    q = _unit(rng.standard_normal((T, Dk)))
    beta = np.ones(T)
    o, fin = _one(run, q, k, v, beta)
    _close(fin, k.T @ v, 1e-13, "recall state K^T V")
    _close(fin.T @ k.T, v.T, 1e-13, "S k_s = v_s")
    expect = np.array([sum((k[s] @ q[t]) * v[s] for s in range(t + 1)) for t in range(T)])
    _close(o, expect, 1e-13, "recall reads")
    g = -0.2 * rng.uniform(0, 1, T)
    o, fin = _one(run, q, k, v, beta, g)
    tail = np.array([np.exp(g[s + 1:].sum()) for s in range(T)])
    _close(fin, k.T @ (tail[:, None] * v), 1e-13, "gated recall state")


def pin_one_token(run):
    """One token from the zero state ([P3] state_input None): S_1 = beta v k^T for any
    gate (the gate acts on the empty state first), and o_1 = beta (k . q) v."""
    rng = np.random.default_rng(15)
    q, k, v, beta, g, _ = _rand_seq(rng, 1, 5, 3, True, False)
    for gg in (None, g, np.array([-2.5])):
        o, fin = _one(run, q, k, v, beta, gg)
        _close(fin, beta[0] * np.outer(k[0], v[0]), 1e-15, "S_1 = beta v k^T")
        _close(o[0], beta[0] * (k[0] @ q[0]) * v[0], 1e-15, "o_1")


def pin_gate_order(run):
    """Two tokens, worked symbolically: with S_1 = b1 v1 k1^T,
    S_2 = a2 S_1 - b2 (a2 S_1 k2 - v2) k2^T  ([P3]: decay, then take up the pair)."""
    rng = np.random.default_rng(16)
    q, k, v, beta, _, _ = _rand_seq(rng, 2, 4, 3, False, False)
    g = np.array([-0.4, -0.9])
    a2 = np.exp(g[1])
    S1 = beta[0] * np.outer(v[0], k[0])
    S2 = a2 * S1 - beta[1] * np.outer(a2 * S1 @ k[1] - v[1], k[1])
    o, fin = _one(run, q, k, v, beta, g)
    _close(fin, S2.T, 1e-14, "two-token gated state")
    _close(o[1], S2 @ q[1], 1e-14, "two-token gated read")


def pin_contraction(run):
    """With v = 0, unit keys, beta in [0, 2] and g <= 0, every step multiplies S by
    exp(g)(I - beta k k^T), whose eigenvalues are exp(g) and exp(g)(1 - beta), all in
    [-1, 1]: ||S_t||_F never grows (the (0, 2) range of [P3] betas).  Checked at every
    prefix through packed sequences; the same inputs with beta = 2.6 must grow."""
    rng = np.random.default_rng(17)
    Dk, Dv, T = 8, 6, 30
    k = _unit(rng.standard_normal((T, Dk)))
    q = _unit(rng.standard_normal((T, Dk)))
    v = np.zeros((T, Dv))
    g = -0.05 * rng.uniform(0, 1, T)
    M0 = rng.standard_normal((Dk, Dv))

    def norms(beta):
        idx = np.concatenate([np.arange(t + 1) for t in range(T)])
        cu = np.concatenate([[0], np.cumsum(np.arange(1, T + 1))])
        N = T
        _, fin = run(q[idx][None, :, None], k[idx][None, :, None], v[idx][None, :, None],
                     beta[idx][None, :, None], g[idx][None, :, None],
                     np.broadcast_to(M0, (N, 1, Dk, Dv)).copy(), cu_seqlens=cu)
        return np.array([np.linalg.norm(fin[t, 0]) for t in range(N)])

    n = norms(rng.uniform(0, 2, T))
    if not (np.all(np.diff(n) <= 1e-12) and n[0] <= np.linalg.norm(M0) + 1e-12):
        raise AssertionError("state norm grew with beta in [0, 2]")
    n_bad = norms(np.full(T, 2.6))
    if not np.any(np.diff(n_bad) > 1e-6):
        raise AssertionError("beta = 2.6 should expand the state")


def pin_linearity(run):
    """For fixed keys, queries, beta and g, the step is affine-linear in (S, v), so the
    outputs and final state are jointly linear in (S_0, V)."""
    rng = np.random.default_rng(18)
    q, k, v1, beta, g, M1 = _rand_seq(rng, 19, 6, 5, True, True, 2.0)
    v2 = rng.standard_normal(v1.shape)
    M2 = rng.standard_normal(M1.shape)
    a, b = 0.75, -1.25
    o1, f1 = _one(run, q, k, v1, beta, g, M1)
    o2, f2 = _one(run, q, k, v2, beta, g, M2)
    o3, f3 = _one(run, q, k, a * v1 + b * v2, beta, g, a * M1 + b * M2)
    _close(o3, a * o1 + b * o2, 1e-12, "linearity o")
    _close(f3, a * f1 + b * f2, 1e-12, "linearity state")


def pin_sgd_step(run):
    """[P2]: the delta rule is one SGD step of size beta on L(S) = 1/2 ||S k - v||^2.
    The gradient is taken here by central finite differences of L (not from its
    formula), so the step's sign and the orientation of the outer product are fixed
    independently of the oracle's algebra."""
    rng = np.random.default_rng(19)
    Dk, Dv = 5, 4
    S = rng.standard_normal((Dv, Dk))
    k = _unit(rng.standard_normal(Dk))
    v = rng.standard_normal(Dv)
    q = _unit(rng.standard_normal(Dk))
    beta = 0.6

    def loss(Sx):
        r = Sx @ k - v
        return 0.5 * r @ r

    grad = np.zeros_like(S)
    h = 1e-5
    for j in range(Dv):
        for i in range(Dk):
            E = np.zeros_like(S)
            E[j, i] = h
            grad[j, i] = (loss(S + E) - loss(S - E)) / (2 * h)
    expect = S - beta * grad
    o, fin = _one(run, q[None], k[None], v[None], np.array([beta]), None, S.T)
    _close(fin, expect.T, 1e-8, "SGD step state")
    _close(o[0], expect @ q, 1e-8, "SGD step read")


def pin_gate_zero_is_plain(run):
    """g = 0 keeps all of the state (exp(0) = 1): the gated rule equals the plain one."""
    rng = np.random.default_rng(20)
    q, k, v, beta, _, M0 = _rand_seq(rng, 21, 6, 6, False, True)
    o1, f1 = _one(run, q, k, v, beta, None, M0)
    o2, f2 = _one(run, q, k, v, beta, np.zeros(21), M0)
    _close(o2, o1, 0, "g=0 output")
    _close(f2, f1, 0, "g=0 state")


def pin_scale(run):
    """The read is linear in the query scale; the state does not depend on it."""
    rng = np.random.default_rng(21)
    q, k, v, beta, g, M0 = _rand_seq(rng, 10, 4, 4, True, True)
    o1, f1 = _one(run, q, k, v, beta, g, M0, scale=1.0)
    o2, f2 = _one(run, q, k, v, beta, g, M0, scale=0.125)
    _close(o2, 0.125 * o1, 1e-15, "scaled read")
    _close(f2, f1, 0, "state independent of scale")


def pin_heads_and_packing(run):
    """Heads and sequences are independent units: a packed multi-head call equals
    per-sequence, per-head calls; value head h reads query/key head h // (Hv/Hqk)
    (consecutive value heads share one repeated query/key head); an empty sequence
    returns its initial state."""
    rng = np.random.default_rng(22)
    Hqk, Hv, Dk, Dv = 2, 6, 5, 3
    lens = [7, 0, 12, 1, 9]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    N = len(lens)
    q = _unit(rng.standard_normal((1, T, Hqk, Dk)))
    k = _unit(rng.standard_normal((1, T, Hqk, Dk)))
    v = rng.standard_normal((1, T, Hv, Dv))
    beta = rng.uniform(0, 2, (1, T, Hv))
    g = -0.2 * rng.uniform(0, 1, (1, T, Hv))
    M0 = rng.standard_normal((N, Hv, Dk, Dv))
    o, fin = run(q, k, v, beta, g, M0, cu_seqlens=cu)
    for n in range(N):
        s, e = cu[n], cu[n + 1]
        for h in range(Hv):
            hq = h // (Hv // Hqk)
            if e == s:
                _close(fin[n, h], M0[n, h], 0, "empty sequence keeps its state")
                continue
            ob, Sb = brute.product_form(q[0, s:e, hq], k[0, s:e, hq], v[0, s:e, h],
                                        beta[0, s:e, h], g[0, s:e, h], M0[n, h].T)
            _close(o[0, s:e, h], ob, 1e-12, f"packed seq {n} head {h} o")
            _close(fin[n, h], Sb.T, 1e-12, f"packed seq {n} head {h} state")


def pin_batch_rows(run):
    """B rows of T tokens are B independent sequences (the same as packing them)."""
    rng = np.random.default_rng(23)
    B, T, H, D = 3, 11, 2, 4
    q = _unit(rng.standard_normal((B, T, H, D)))
    k = _unit(rng.standard_normal((B, T, H, D)))
    v = rng.standard_normal((B, T, H, D))
    beta = rng.uniform(0, 1, (B, T, H))
    o, fin = run(q, k, v, beta)
    for b in range(B):
        for h in range(H):
            ob, Sb = brute.product_form(q[b, :, h], k[b, :, h], v[b, :, h], beta[b, :, h])
            _close(o[b, :, h], ob, 1e-12, "batch row o")
            _close(fin[b, h], Sb.T, 1e-12, "batch row state")


# ------------------------------------------------ normalisation inside the rule
# [P1] class text: queries and keys are L2-normalised; [P2] block flowchart: "L2 Norm" on
# q and k right before the "Delta Rule" box.  Reading: x / sqrt(sum x^2 + eps).

def _raw_qk(rng, shape, lo=0.05, hi=20.0):
    """Gaussian vectors with per-vector magnitudes spread over [lo, hi]."""
    x = _unit(rng.standard_normal(shape))
    return x * rng.uniform(lo, hi, shape[:-1] + (1,))


def pin_l2norm_is_library_normalise(run):
    """With eps = 0, normalising inside the rule equals handing the rule inputs that
    numpy has normalised (numpy.linalg.norm), over GQA heads, packed sequences, gate,
    initial state and beta in (0, 2)."""
    rng = np.random.default_rng(31)
    Hqk, Hv, Dk, Dv = 2, 4, 6, 3
    lens = [9, 0, 5]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = _raw_qk(rng, (1, T, Hqk, Dk))
    k = _raw_qk(rng, (1, T, Hqk, Dk))
    v = rng.standard_normal((1, T, Hv, Dv))
    beta = rng.uniform(0, 2, (1, T, Hv))
    g = -0.2 * rng.uniform(0, 1, (1, T, Hv))
    M0 = rng.standard_normal((len(lens), Hv, Dk, Dv))
    o1, f1 = run(q, k, v, beta, g, M0, cu_seqlens=cu, qk_l2norm=True, eps=0.0)
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    o2, f2 = run(qn, kn, v, beta, g, M0, cu_seqlens=cu)
    _close(o1, o2, 1e-13, "normalised in the rule vs by numpy: o")
    _close(f1, f2, 1e-13, "normalised in the rule vs by numpy: state")


def pin_l2norm_eps_one_token(run):
    """One token from the zero state with k = c u, q = d w (u, w unit): the normalised
    key is c u / sqrt(c^2 + eps), so S_1 = beta v k^T / sqrt(c^2 + eps) and
    o_1 = beta (u.w) c d / (sqrt(c^2 + eps) sqrt(d^2 + eps)) v.  Small c and d make eps
    visible (it sits under the square root)."""
    rng = np.random.default_rng(32)
    Dk, Dv, eps = 5, 3, 1e-6
    u = _unit(rng.standard_normal(Dk))
    w = _unit(rng.standard_normal(Dk))
    c, d, b = 2e-3, 3e-3, 0.7
    v = rng.standard_normal(Dv)
    o, fin = run((d * w).reshape(1, 1, 1, Dk), (c * u).reshape(1, 1, 1, Dk),
                 v.reshape(1, 1, 1, Dv), np.full((1, 1, 1), b), qk_l2norm=True, eps=eps)
    nk, nq = np.sqrt(c * c + eps), np.sqrt(d * d + eps)
    _close(fin.reshape(Dk, Dv), b * np.outer(c * u / nk, v), 1e-14, "one-token state")
    _close(o.reshape(Dv), b * (u @ w) * c * d / (nk * nq) * v, 1e-14, "one-token read")


def pin_l2norm_scale_free(run):
    """Normalised inside the rule, q_t and k_t count only by direction (eps = 0): any
    positive per-token rescaling leaves o and the state unchanged; a zero key (eps > 0)
    leaves the state only decayed."""
    rng = np.random.default_rng(33)
    T, Dk, Dv = 8, 4, 5
    q, k, v, beta, g, M0 = _rand_seq(rng, T, Dk, Dv, True, True)
    cq = rng.uniform(0.1, 10, (T, 1))
    ck = rng.uniform(0.1, 10, (T, 1))
    norm = dict(qk_l2norm=True, eps=0.0)
    o1, f1 = _one(lambda *a, **kw: run(*a, **kw, **norm), q, k, v, beta, g, M0)
    o2, f2 = _one(lambda *a, **kw: run(*a, **kw, **norm), cq * q, ck * k, v, beta, g, M0)
    _close(o2, o1, 1e-13, "rescaled q, k: o")
    _close(f2, f1, 1e-13, "rescaled q, k: state")
    z = np.zeros((1, Dk))
    o3, f3 = _one(lambda *a, **kw: run(*a, **kw, qk_l2norm=True, eps=1e-6),
                  q[:1], z, v[:1], beta[:1], g[:1], M0)
    _close(f3, np.exp(g[0]) * M0, 1e-15, "zero key: state only decayed")


# ------------------------------------------------------- gates per key channel
# [P3] ChannelGates [batch, seq, heads, key_dim] (the KDA variant).  Reading: key channel i
# of the state keeps exp(g_t[i]): S'_t = S_{t-1} diag(exp(g_t)).

def pin_channel_gates_product_form(run):
    """Channel gates against the explicit-matrix product form with diag(exp(g_t)), d_k != d_v,
    beta in (0, 2), an initial state."""
    rng = np.random.default_rng(41)
    T, Dk, Dv = 9, 5, 3
    q, k, v, beta, _, M0 = _rand_seq(rng, T, Dk, Dv, False, True, beta_hi=2.0)
    g = -0.5 * rng.uniform(0, 1, (T, Dk))
    o, fin = run(q.reshape(1, T, 1, Dk), k.reshape(1, T, 1, Dk), v.reshape(1, T, 1, Dv),
                 beta.reshape(1, T, 1), g.reshape(1, T, 1, Dk), M0.reshape(1, 1, Dk, Dv))
    ob, Sb = brute.product_form(q, k, v, beta, g, M0.T)
    _close(o.reshape(T, Dv), ob, 1e-13, "channel gates: o")
    _close(fin.reshape(Dk, Dv), Sb.T, 1e-13, "channel gates: state")


def pin_channel_gates_uniform_are_the_head_gate(run):
    """The same gate on every key channel is the one-gate-per-head rule."""
    rng = np.random.default_rng(42)
    T, Dk, Dv = 12, 4, 6
    q, k, v, beta, g, M0 = _rand_seq(rng, T, Dk, Dv, True, True)
    gc = np.repeat(g[:, None], Dk, axis=1)
    shp = lambda x, *d: x.reshape(1, T, 1, *d)
    o1, f1 = run(shp(q, Dk), shp(k, Dk), shp(v, Dv), beta.reshape(1, T, 1), gc.reshape(1, T, 1, Dk),
                 M0.reshape(1, 1, Dk, Dv))
    o2, f2 = _one(run, q, k, v, beta, g, M0)
    _close(o1.reshape(T, Dv), o2, 1e-14, "uniform channel gates: o")
    _close(f1.reshape(Dk, Dv), f2, 1e-14, "uniform channel gates: state")


def pin_channel_gates_decay_only(run):
    """beta = 0: key channel i of the state is scaled by exp(sum_s g_s[i]) and nothing else
    happens (closed form, d_k != d_v); the read is S_t q_t."""
    rng = np.random.default_rng(43)
    T, Dk, Dv = 7, 3, 5
    q, k, v, _, _, M0 = _rand_seq(rng, T, Dk, Dv, False, True)
    g = -rng.uniform(0, 0.7, (T, Dk))
    o, fin = run(q.reshape(1, T, 1, Dk), k.reshape(1, T, 1, Dk), v.reshape(1, T, 1, Dv),
                 np.zeros((1, T, 1)), g.reshape(1, T, 1, Dk), M0.reshape(1, 1, Dk, Dv))
    cum = np.cumsum(g, axis=0)
    want_o = np.stack([(np.exp(cum[t])[:, None] * M0).T @ q[t] for t in range(T)])
    _close(fin.reshape(Dk, Dv), np.exp(cum[-1])[:, None] * M0, 1e-15, "decay-only state")
    _close(o.reshape(T, Dv), want_o, 1e-15, "decay-only read")


def pin_channel_gates_heads_and_packing(run):
    """Channel gates [1, T, Hv, Dk] over GQA heads and packed sequences: each (sequence,
    value head) unit equals the product form with its own gate rows."""
    rng = np.random.default_rng(44)
    Hqk, Hv, Dk, Dv = 1, 3, 4, 2
    lens = [6, 0, 9]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = _unit(rng.standard_normal((1, T, Hqk, Dk)))
    k = _unit(rng.standard_normal((1, T, Hqk, Dk)))
    v = rng.standard_normal((1, T, Hv, Dv))
    beta = rng.uniform(0, 2, (1, T, Hv))
    g = -0.4 * rng.uniform(0, 1, (1, T, Hv, Dk))
    M0 = rng.standard_normal((len(lens), Hv, Dk, Dv))
    o, fin = run(q, k, v, beta, g, M0, cu_seqlens=cu)
    for n in range(len(lens)):
        s_, e_ = cu[n], cu[n + 1]
        for h in range(Hv):
            if e_ == s_:
                _close(fin[n, h], M0[n, h], 0, "empty sequence keeps its state")
                continue
            ob, Sb = brute.product_form(q[0, s_:e_, 0], k[0, s_:e_, 0], v[0, s_:e_, h],
                                        beta[0, s_:e_, h], g[0, s_:e_, h], M0[n, h].T)
            _close(o[0, s_:e_, h], ob, 1e-12, f"channel gates seq {n} head {h}: o")
            _close(fin[n, h], Sb.T, 1e-12, f"channel gates seq {n} head {h}: state")


ALL_PINS = [pin_hand_worked, pin_product_form, pin_retrieve_interpolate, pin_beta_zero,
            pin_exact_recall, pin_one_token, pin_gate_order, pin_contraction, pin_linearity,
            pin_sgd_step, pin_gate_zero_is_plain, pin_scale, pin_heads_and_packing,
            pin_batch_rows, pin_l2norm_is_library_normalise, pin_l2norm_eps_one_token,
            pin_l2norm_scale_free, pin_channel_gates_product_form,
            pin_channel_gates_uniform_are_the_head_gate, pin_channel_gates_decay_only,
            pin_channel_gates_heads_and_packing]
