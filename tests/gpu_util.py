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


def per_unit_rel(o, o_ref, s, s_ref, x: DeltaInputs):
    """Relative L2 of every (sequence, value head): the output over that sequence's tokens
    and the final state.  Returns (worst output error, worst state error, where)."""
    bounds = x.seq_bounds()
    Hv, Dv = x.Hv, x.Dv
    of = np.asarray(o, dtype=np.float64).reshape(-1, Hv, Dv)
    rf = np.asarray(o_ref, dtype=np.float64).reshape(-1, Hv, Dv)
    worst_o = worst_s = 0.0
    where = None
    for n in range(len(bounds) - 1):
        a, b = int(bounds[n]), int(bounds[n + 1])
        for h in range(Hv):
            eo = rel_l2(of[a:b, h], rf[a:b, h]) if b > a else 0.0
            es = rel_l2(s[n, h], s_ref[n, h])
            if eo > worst_o or es > worst_s:
                where = (n, h, b - a)
            worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
    return worst_o, worst_s, where


def log_errors(case: str, **errors):
    """Append one case's measured errors to parity_errors.jsonl in the output folder of the
    run (DN_OUTPUT_DIR, by default the repository's untracked output folder)."""
    import json
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = os.environ.get("DN_OUTPUT_DIR", os.path.join(root, "gpurun_out"))
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(out, "parity_errors.jsonl"), "a") as f:
        f.write(json.dumps({"case": case, **{k: (float(v) if isinstance(v, (float, np.floating))
                                                  else v) for k, v in errors.items()}}) + "\n")
