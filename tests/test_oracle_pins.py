"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle import brute
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(oracle.recurrent)


@pytest.mark.parametrize("form", [brute.product_form, brute.retrieve_interpolate_form])
def test_brute_forms_on_hand_worked(form):
    """The two brute-force twins reproduce the hand-worked examples too (so they are
    pinned independently of the oracle they are compared with)."""
    from tests.golden import load_hand_worked
    for name, c in load_hand_worked().items():
        o, S = form(c["q"], c["k"], c["v"], c["beta"], c["g"],
                    None if c["init"] is None else c["init"].T)
        np.testing.assert_allclose(o, c["o"], atol=1e-13, err_msg=name)
        np.testing.assert_allclose(S.T, c["final"], atol=1e-13, err_msg=name)


def test_config1_against_product_form():
    """The smallest workload (plain rule, B1 H2 T64 d16, fp32 inputs) in full against the
    explicit-matrix product form."""
    from synth import make_config
    x = make_config(1)
    f = x.f64()
    o, fin = oracle.recurrent(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"])
    for h in range(x.Hv):
        ob, Sb = brute.product_form(f["q"][0, :, h], f["k"][0, :, h], f["v"][0, :, h],
                                    f["beta"][0, :, h])
        np.testing.assert_allclose(o[0, :, h], ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(fin[0, h], Sb.T, rtol=0, atol=1e-12)


def test_bad_arguments():
    q = np.zeros((1, 4, 2, 3))
    v = np.zeros((1, 4, 3, 3))
    with pytest.raises(ValueError):       # Hv not a multiple of Hqk
        oracle.recurrent(q, q, v, np.zeros((1, 4, 3)))
    v = np.zeros((1, 4, 2, 3))
    with pytest.raises(ValueError):       # packed batch must end at T
        oracle.recurrent(q, q, v, np.zeros((1, 4, 2)), cu_seqlens=np.array([0, 3]))
    with pytest.raises(ValueError):       # decreasing offsets
        oracle.recurrent(q, q, v, np.zeros((1, 4, 2)), cu_seqlens=np.array([0, 3, 2, 4]))
    with pytest.raises(ValueError):       # init shape
        oracle.recurrent(q, q, v, np.zeros((1, 4, 2)), init=np.zeros((1, 2, 3, 4)))


def test_threads_reported():
    assert oracle.max_threads() >= 1


@pytest.mark.parametrize("gate", [None, "head", "key"])
def test_per_token_states_at_every_prefix(gate):
    """brute.per_token_states (the checker of the GPU state trace) against the oracle at
    every prefix: the T prefixes of one sequence packed as T sequences of lengths 1..T
    into one oracle call, whose final states must be the trace's states, token by token.
    Gates per head, per key channel, or none; d_k != d_v, beta in (0, 2), initial state."""
    rng = np.random.default_rng(11)
    T, Dk, Dv = 23, 5, 7
    k = rng.standard_normal((T, Dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, Dv))
    beta = 2.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    g = None
    if gate == "head":
        g = -0.3 * np.log1p(np.exp(rng.standard_normal(T)))
    elif gate == "key":
        g = -0.3 * np.log1p(np.exp(rng.standard_normal((T, Dk))))
    S0 = rng.standard_normal((Dv, Dk)) * 0.5
    trace = brute.per_token_states(k, v, beta, g, S0)
    assert trace.shape == (T, Dv, Dk)
    # packed prefixes: sequence t holds tokens 0..t
    idx = np.concatenate([np.arange(t + 1) for t in range(T)])
    cu = np.concatenate([[0], np.cumsum(np.arange(1, T + 1))])
    pk = k[idx][None, :, None, :]
    pv = v[idx][None, :, None, :]
    pb = beta[idx][None, :, None]
    pg = None
    if g is not None:
        pg = g[idx][None, :, None] if g.ndim == 1 else g[idx][None, :, None, :]
    init = np.broadcast_to(S0.T, (T, 1, Dk, Dv)).copy()
    _, fin = oracle.recurrent(pk, pk, pv, pb, pg, init, cu_seqlens=cu)
    for t in range(T):
        np.testing.assert_allclose(trace[t].T, fin[t, 0], rtol=0, atol=1e-12, err_msg=f"token {t}")
    # and the last state is the product form's final state
    _, S_T = brute.product_form(k, k, v, beta, g, S0)
    np.testing.assert_allclose(trace[-1], S_T, rtol=0, atol=1e-13)
