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
