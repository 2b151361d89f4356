"""fp64 CPU oracle of the (gated) delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  It shares no code with the HIP library and the HIP
library never calls it.

* :func:`recurrent` -- the oracle of record: ``dn_oracle.c``, a token-by-token fp64
  recurrence (error-correction form of the delta rule, with the gate applied first
  and the read after the write), OpenMP over independent (sequence, value head)
  pairs.
* :mod:`oracle.brute` -- tiny-input twins written from the other readings the pages
  give of the same update (explicit product form, retrieve/interpolate form).

Parity status: pinned.  ``tests/test_oracle_pins.py`` checks the oracle against the
pages' other stated forms, closed forms (exact recall, one token, decay only),
invariants (contraction for beta in [0, 2], linearity, the SGD-step reading via a
finite-difference gradient) and hand-worked examples in ``tests/golden/``;
``tests/test_oracle_mutants.py`` plants plausible mistakes in copies of the source
and checks that the pins catch every one.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "dn_oracle.c")
LIB = os.path.join(_HERE, "libdn_oracle.so")
_libs = {}

__all__ = ["build", "compile_source", "recurrent", "max_threads", "SRC", "LIB"]


def compile_source(src: str, out: str, werror: bool = True) -> str:
    """gcc -O2 -fopenmp shared build of one oracle source file."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall"]
    cmd += ["-Werror"] if werror else ["-w"]
    cmd += [src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile ``dn_oracle.c`` into ``oracle/libdn_oracle.so``."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        compile_source(SRC, LIB)
        _libs.pop(LIB, None)
    return LIB


def _load(lib_path: Optional[str] = None):
    """Bind the oracle library, or another build of the same source at ``lib_path``
    (the mutation tests plant mistakes in copies of ``dn_oracle.c``)."""
    path = LIB if lib_path is None else lib_path
    if path not in _libs:
        if lib_path is None:
            build(force=False)
        lib = ctypes.CDLL(path)
        d = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.dn_oracle_fwd.argtypes = [i64, ctypes.POINTER(i64), i64, i64, i64, i64,
                                      d, d, d, d, d, i64, d, ctypes.c_double, ctypes.c_int,
                                      ctypes.c_double, d, d, ctypes.c_int]
        lib.dn_oracle_fwd.restype = ctypes.c_int
        lib.dn_oracle_max_threads.argtypes = []
        lib.dn_oracle_max_threads.restype = ctypes.c_int
        _libs[path] = lib
    return _libs[path]


def max_threads() -> int:
    """OpenMP threads the oracle uses by default on this host."""
    return int(_load().dn_oracle_max_threads())


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrent(q: np.ndarray, k: np.ndarray, v: np.ndarray, beta: np.ndarray,
              g: Optional[np.ndarray] = None, init: Optional[np.ndarray] = None,
              cu_seqlens: Optional[np.ndarray] = None, scale: float = 1.0,
              nthreads: int = 0, lib_path: Optional[str] = None,
              qk_l2norm: bool = False, eps: float = 1e-6
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Run the token-by-token delta rule in fp64.

    With ``qk_l2norm`` every q_t and k_t is first replaced by
    ``x / sqrt(sum(x**2) + eps)`` (normalisation inside the rule).

    q, k: ``[B, T, Hqk, Dk]``; v: ``[B, T, Hv, Dv]``; beta: ``[B, T, Hv]``; g: ``[B, T, Hv]``
    (one log decay per head) or ``[B, T, Hv, Dk]`` (per key channel);
    init: ``[N, Hv, Dk, Dv]`` (key-major state) or None.  With ``cu_seqlens``
    (``[N + 1]``) the B*T tokens are N packed sequences, else each of the B rows is one
    sequence.  Returns ``(o [B, T, Hv, Dv], final [N, Hv, Dk, Dv])`` in fp64.
    Raises ValueError on inconsistent shapes.
    """
    lib = _load(lib_path)
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    beta = np.ascontiguousarray(beta, dtype=np.float64)
    if q.ndim != 4 or k.shape != q.shape or v.ndim != 4 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [B, T, Hqk, Dk] and v [B, T, Hv, Dv]")
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    if beta.shape != (B, T, Hv):
        raise ValueError("beta must be [B, T, Hv]")
    gdim = 1
    if g is not None:
        g = np.ascontiguousarray(g, dtype=np.float64)
        if g.shape == (B, T, Hv, Dk):
            gdim = Dk
        elif g.shape != (B, T, Hv):
            raise ValueError("g must be [B, T, Hv] or [B, T, Hv, Dk]")
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        if B != 1 or cu.ndim != 1 or len(cu) < 1 or cu[-1] != T:
            raise ValueError("packed sequences need B == 1 and cu_seqlens[-1] == T")
    N = len(cu) - 1
    if init is not None:
        init = np.ascontiguousarray(init, dtype=np.float64)
        if init.shape != (N, Hv, Dk, Dv):
            raise ValueError("init must be [N, Hv, Dk, Dv]")
    o = np.zeros((B, T, Hv, Dv), dtype=np.float64)
    final = np.zeros((N, Hv, Dk, Dv), dtype=np.float64)
    rc = lib.dn_oracle_fwd(N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                           Hqk, Hv, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                           gdim, _ptr(init), float(scale), int(bool(qk_l2norm)), float(eps),
                           _ptr(o), _ptr(final), int(nthreads))
    if rc != 0:
        raise ValueError(f"dn_oracle_fwd rejected its arguments (rc={rc})")
    return o, final
