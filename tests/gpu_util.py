"""Helpers for the GPU tests: move generated inputs to the device, run the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import DeltaInputs


def dev_tensor(x, device="cuda"):
    """Host array -> device tensor; uint16 arrays are bf16 bit patterns."""
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def to_inputs(x: DeltaInputs, device="cuda"):
    return dict(q=dev_tensor(x.q, device), k=dev_tensor(x.k, device), v=dev_tensor(x.v, device),
                beta=dev_tensor(x.beta, device), g=dev_tensor(x.g, device),
                init=dev_tensor(x.init, device),
                cu=None if x.cu_seqlens is None else dev_tensor(x.cu_seqlens.astype(np.int32), device))


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_oracle(x: DeltaInputs, scale=1.0):
    f = x.f64()
    return oracle.recurrent(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"],
                            x.cu_seqlens, scale=scale)


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    d = np.linalg.norm(b.ravel())
    return float(np.linalg.norm((a - b).ravel()) / (d if d > 0 else 1.0))


def tol(x: DeltaInputs) -> float:
    """Relative-L2 bar on outputs and final states: 1e-4 for fp32 inputs, 1e-2 for bf16."""
    return 1e-4 if x.dtype == "f32" else 1e-2
