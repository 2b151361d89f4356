"""fp64 reference of the readout epilogue -- TEST INFRASTRUCTURE ONLY (see
``oracle/__init__.py``): only the tests, the smoke check and the benchmark's CPU leg may
import it, and the HIP library never calls it.

The step after the rule, per (token, value head), over the d_v readout o:

* the frankenstein "DeltaNet Attention" page (attributes ``norm`` and ``g_proj``): a
  layer normalisation of the recurrent readout, then the silu-gated output gate;
* the mutichung "DeltaNet" page (block flowchart): the Delta Rule box feeds an RMSNorm
  box, then the output projection.

Reading: the normalisation runs over the d_v entries of one head's readout, with a weight
(and, for the layer norm, a bias) of length d_v shared by the heads; the gate z has the
readout's shape and multiplies elementwise as silu(z) = z / (1 + exp(-z)).  Both norms
put eps inside the square root; the layer norm uses the biased variance.

    rms:    y = o / sqrt(mean(o^2) + eps) * w
    layer:  y = (o - mean(o)) / sqrt(mean((o - mean(o))^2) + eps) * w + b
    gated:  y <- y * silu(z)
"""
from __future__ import annotations

from typing import Optional

import numpy as np

__all__ = ["norm_gate", "silu"]


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def norm_gate(o: np.ndarray, kind: str = "rms", eps: float = 1e-6,
              weight: Optional[np.ndarray] = None, bias: Optional[np.ndarray] = None,
              gate: Optional[np.ndarray] = None) -> np.ndarray:
    """o ``[..., Dv]`` -> y ``[..., Dv]`` in fp64 (see the module docstring)."""
    o = np.asarray(o, dtype=np.float64)
    Dv = o.shape[-1]
    w = np.ones(Dv) if weight is None else np.asarray(weight, dtype=np.float64)
    if kind == "rms":
        y = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps) * w
    elif kind == "layer":
        c = o - np.mean(o, axis=-1, keepdims=True)
        y = c / np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + eps) * w
        if bias is not None:
            y = y + np.asarray(bias, dtype=np.float64)
    else:
        raise ValueError(f"unknown norm kind {kind!r}")
    if gate is not None:
        y = y * silu(gate)
    return y
