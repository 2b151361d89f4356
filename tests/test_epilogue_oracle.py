"""Pins of the readout-epilogue reference (oracle/epilogue.py) against what the pages and
the mathematics fix, and against library routines (CPU only)."""
import numpy as np
import pytest
import torch

from oracle.epilogue import norm_gate, silu


def test_rms_matches_torch_rms_norm():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((5, 3, 16))
    w = rng.uniform(0.5, 2, 16)
    want = torch.nn.functional.rms_norm(torch.from_numpy(o), (16,), torch.from_numpy(w), eps=1e-5)
    np.testing.assert_allclose(norm_gate(o, "rms", 1e-5, w), want.numpy(), rtol=1e-13, atol=1e-13)


def test_layer_matches_torch_layer_norm():
    rng = np.random.default_rng(2)
    o = 3 + rng.standard_normal((4, 2, 32))
    w, b = rng.uniform(0.5, 2, 32), rng.standard_normal(32)
    want = torch.nn.functional.layer_norm(torch.from_numpy(o), (32,), torch.from_numpy(w),
                                          torch.from_numpy(b), eps=1e-5)
    np.testing.assert_allclose(norm_gate(o, "layer", 1e-5, w, b), want.numpy(), rtol=1e-12, atol=1e-12)


def test_silu_matches_torch_and_closed_forms():
    z = np.linspace(-8, 8, 33)
    np.testing.assert_allclose(silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(),
                               rtol=1e-14, atol=1e-15)
    assert silu(np.array(0.0)) == 0.0
    np.testing.assert_allclose(silu(np.array(1.0)), 1.0 / (1.0 + np.exp(-1.0)), rtol=1e-15)


def test_invariants():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((6, 8))
    # unit weight, no gate, eps = 0: RMS 1 (rms); mean 0 and variance 1 (layer)
    y = norm_gate(o, "rms", 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    y = norm_gate(o, "layer", 0.0)
    np.testing.assert_allclose(np.mean(y, axis=-1), 0.0, atol=1e-14)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-14)
    # scale-free in o for eps = 0 (positive scale); layer norm also shift-free
    for kind in ("rms", "layer"):
        np.testing.assert_allclose(norm_gate(7.5 * o, kind, 0.0), norm_gate(o, kind, 0.0), rtol=1e-13)
    np.testing.assert_allclose(norm_gate(o + 4.0, "layer", 0.0), norm_gate(o, "layer", 0.0), atol=1e-13)
    # a zero gate zeroes the output; the gate multiplies elementwise
    z = rng.standard_normal(o.shape)
    assert np.all(norm_gate(o, "rms", 1e-6, gate=np.zeros_like(o)) == 0)
    np.testing.assert_allclose(norm_gate(o, "rms", 1e-6, gate=z), norm_gate(o, "rms", 1e-6) * silu(z), rtol=1e-15)


def test_two_entry_closed_form():
    """o = (a, -a): mean 0, mean square a^2, so rms and layer agree:
    y = (a, -a) / sqrt(a^2 + eps) * w (+ b)."""
    a, eps = 0.3, 1e-2
    o = np.array([a, -a])
    w, b = np.array([2.0, 0.5]), np.array([0.25, -1.0])
    want = np.array([a, -a]) / np.sqrt(a * a + eps) * w
    np.testing.assert_allclose(norm_gate(o, "rms", eps, w), want, rtol=1e-15)
    np.testing.assert_allclose(norm_gate(o, "layer", eps, w, b), want + b, rtol=1e-15)


def test_bad_kind():
    with pytest.raises(ValueError):
        norm_gate(np.zeros(4), "batch")
