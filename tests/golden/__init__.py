"""Parser for the hand-worked fixtures in this folder."""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def load_hand_worked(path=os.path.join(HERE, "hand_worked.txt")):
    cases, cur = {}, None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("case "):
                cur = {}
                cases[line[5:].strip()] = cur
                continue
            key, val = line.split(":", 1)
            val = val.strip()
            cur[key.strip()] = None if val == "none" else np.array(
                [float(x) for x in val.split()], dtype=np.float64)
    out = {}
    for name, c in cases.items():
        Dk, Dv, T = (int(x) for x in c["dims"])
        out[name] = dict(
            Dk=Dk, Dv=Dv, T=T,
            q=c["q"].reshape(T, Dk), k=c["k"].reshape(T, Dk), v=c["v"].reshape(T, Dv),
            beta=c["beta"].reshape(T), g=None if c["g"] is None else c["g"].reshape(T),
            init=None if c["init"] is None else c["init"].reshape(Dk, Dv),
            o=c["o"].reshape(T, Dv), final=c["final"].reshape(Dk, Dv))
    return out
