"""Seeded synthetic inputs for the delta-rule mixer.

This module is shared by the fp64 oracle and the HIP path, so it holds no part of
the delta rule itself: it only draws random numbers, shapes them like the tensors
a gated DeltaNet mixer hands to its delta-rule kernel, and casts them.

Shapes follow the tensor accessors of the nnterp "linear_attention" page
(queries/keys ``[batch, seq, heads, key_dim]``, values ``[batch, seq, heads,
value_dim]``, decays and betas ``[batch, seq, heads]`` in float32).  The
preconditions the pages put on those inputs are applied here:

* q and k are L2-normalised per (token, head) before the rule (frankenstein
  DeltaNetAttention docstring; the L2 Norm box of the DeltaNet block flowchart on
  the mutichung garden page), in fp64 and before any cast -- unless the case asks
  for raw q and k (``qk_raw``), for calls that normalise inside the rule;
* beta is a sigmoid output in (0, 1), or twice that, in (0, 2), for the
  negative-eigenvalue variant (nnterp ``betas``);
* the log decay g is non-positive (nnterp ``decays``), drawn as
  ``-c * softplus(z)``, one per head or one per key channel (``ChannelGates``).

Draw order per case, from one ``numpy.random.default_rng(seed)``: q, k, v, z_beta,
z_g, initial state, then the cut points of a packed (varlen) batch.  Normal draws
are fp64.  bf16 tensors are returned as uint16 bit patterns, rounded to nearest
even from the fp32 value; both sides of every comparison consume those same bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "DeltaInputs", "make_case", "make_config", "CONFIG_NAMES", "make_epilogue_inputs",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "to_f64",
]


# ----------------------------------------------------------------------------- casts

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32, exact."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_f64(x: Optional[np.ndarray], dtype: str = "f32") -> Optional[np.ndarray]:
    """Exact upcast of a generated tensor (fp32 values or bf16 bits) to fp64."""
    if x is None:
        return None
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------- inputs

@dataclass
class DeltaInputs:
    """One delta-rule call's inputs, as host arrays.

    Layout is token-major: q, k ``[B, T, Hqk, Dk]``, v ``[B, T, Hv, Dv]``, beta and g
    ``[B, T, Hv]`` fp32 (g ``[B, T, Hv, Dk]`` for gates per key channel).  A packed batch has ``B == 1``, ``T`` = total tokens and
    ``cu_seqlens`` (int32, ``[N + 1]``).  ``init`` is ``[N, Hv, Dk, Dv]`` fp32, the
    state stored key-major (the transpose of the value-by-key map S), or None for a
    fresh prompt.  q/k/v are fp32 when ``dtype == "f32"`` and bf16 bit patterns
    (uint16) when ``dtype == "bf16"``.
    """

    name: str
    dtype: str
    B: int
    T: int
    Hqk: int
    Hv: int
    Dk: int
    Dv: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    beta: np.ndarray
    g: Optional[np.ndarray]
    init: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]
    chunk: int = 64
    decode: bool = False
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return self.B if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def seq_bounds(self) -> np.ndarray:
        """Token offsets [N + 1] of each sequence in the flattened B*T token axis."""
        if self.cu_seqlens is not None:
            return np.asarray(self.cu_seqlens, dtype=np.int64)
        return np.arange(self.B + 1, dtype=np.int64) * self.T

    def f64(self) -> dict:
        """Every tensor upcast exactly to fp64 (None stays None)."""
        return dict(q=to_f64(self.q), k=to_f64(self.k), v=to_f64(self.v),
                    beta=to_f64(self.beta), g=to_f64(self.g), init=to_f64(self.init))


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def _softplus(z: np.ndarray) -> np.ndarray:
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def _cast(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(x32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_case(*, B: int = 1, T: int = 64, Hqk: int = 2, Hv: Optional[int] = None,
              Dk: int = 16, Dv: Optional[int] = None, dtype: str = "f32",
              beta_scale: float = 1.0, g_scale: Optional[float] = None,
              init_std: Optional[float] = None, seqlens: Optional[Sequence[int]] = None,
              num_seqs_cut: Optional[int] = None, chunk: int = 64, seed: int = 0,
              name: str = "case", decode: bool = False, qk_raw: bool = False,
              g_per_key: bool = False) -> DeltaInputs:
    """Draw one case.

    ``beta = beta_scale * sigmoid(z)``; ``g = -g_scale * softplus(z)`` or no decay when
    ``g_scale`` is None; ``init ~ N(0, init_std^2)`` per sequence or a zero (None) state.
    A packed batch is asked for either with explicit ``seqlens`` or with
    ``num_seqs_cut`` = N, which cuts T at N - 1 distinct points drawn uniformly
    without replacement from {1, ..., T - 1}.  With ``qk_raw`` q and k are the raw
    N(0, 1) draws (norm about sqrt(Dk)), not normalised.  With ``g_per_key`` the log decay
    is drawn per key channel, ``[B, T, Hv, Dk]`` (the nnterp page's ChannelGates).
    """
    Hv = Hqk if Hv is None else Hv
    Dv = Dk if Dv is None else Dv
    if Hv % Hqk:
        raise ValueError("Hv must be a multiple of Hqk")
    rng = np.random.default_rng(seed)
    if seqlens is not None or num_seqs_cut is not None:
        if B != 1:
            raise ValueError("a packed batch has B == 1")
        if seqlens is not None:
            T = int(sum(seqlens))
    shape_qk = (B, T, Hqk, Dk)
    q = rng.standard_normal(shape_qk)
    k = rng.standard_normal(shape_qk)
    if not qk_raw:
        q = _l2_normalise(q)
        k = _l2_normalise(k)
    v = rng.standard_normal((B, T, Hv, Dv))
    beta = (beta_scale * _sigmoid(rng.standard_normal((B, T, Hv)))).astype(np.float32)
    g = None
    if g_scale is not None:
        gshape = (B, T, Hv, Dk) if g_per_key else (B, T, Hv)
        g = (-g_scale * _softplus(rng.standard_normal(gshape))).astype(np.float32)
    cu = None
    if seqlens is not None:
        cu = np.concatenate([[0], np.cumsum(np.asarray(seqlens, dtype=np.int64))])
    N = B if (seqlens is None and num_seqs_cut is None) else (
        len(seqlens) if seqlens is not None else num_seqs_cut)
    init = None
    if init_std is not None:
        init = (init_std * rng.standard_normal((N, Hv, Dk, Dv))).astype(np.float32)
    if num_seqs_cut is not None and seqlens is None:
        cuts = np.sort(rng.choice(np.arange(1, T), size=num_seqs_cut - 1, replace=False))
        cu = np.concatenate([[0], cuts, [T]])
    return DeltaInputs(
        name=name, dtype=dtype, B=B, T=T, Hqk=Hqk, Hv=Hv, Dk=Dk, Dv=Dv,
        q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype), beta=beta, g=g,
        init=init, cu_seqlens=None if cu is None else cu.astype(np.int32),
        chunk=chunk, decode=decode, meta={"qk_raw": qk_raw})


CONFIG_NAMES = {
    1: "plain delta rule B1 H2 T64 d16 fp32",
    2: "DeltaNet prefill B4 H16 T2048 d128 bf16",
    3: "gated GQA prefill B2 16->32 heads T8192 d128 bf16",
    4: "gated decode step 256 seqs x 32 heads d128 bf16",
    5: "varlen gated prefill 8 seqs sum 32768 32 heads d128 bf16, beta in (0,2)",
}


def make_config(i: int, seed: int = 0) -> DeltaInputs:
    """The five workloads the mixer is measured and checked on."""
    if i == 1:
        return make_case(B=1, T=64, Hqk=2, Dk=16, dtype="f32", seed=seed,
                         name=CONFIG_NAMES[1])
    if i == 2:
        return make_case(B=4, T=2048, Hqk=16, Dk=128, dtype="bf16", seed=seed,
                         name=CONFIG_NAMES[2])
    if i == 3:
        return make_case(B=2, T=8192, Hqk=16, Hv=32, Dk=128, dtype="bf16", g_scale=0.1,
                         seed=seed, name=CONFIG_NAMES[3])
    if i == 4:
        return make_case(B=256, T=1, Hqk=32, Dk=128, dtype="bf16", g_scale=0.1,
                         init_std=0.02, seed=seed, name=CONFIG_NAMES[4], decode=True)
    if i == 5:
        return make_case(B=1, T=32768, Hqk=32, Dk=128, dtype="bf16", beta_scale=2.0,
                         g_scale=0.05, init_std=0.02, num_seqs_cut=8, seed=seed,
                         name=CONFIG_NAMES[5])
    raise ValueError(f"no config {i}")


def make_epilogue_inputs(shape, dtype: str = "bf16", seed: int = 0, offset: float = 0.5) -> dict:
    """Seeded inputs of the readout epilogue: a readout ``o`` of ``shape`` (``[..., Dv]``,
    N(offset, 1)), an output gate ``gate`` of the same shape (N(0, 1)), both cast like
    q/k/v (fp32 values or bf16 bit patterns), and fp32 ``weight`` (U(0.5, 1.5)) and
    ``bias`` (N(0, 0.1^2)) of length Dv.  Draw order: o, gate, weight, bias."""
    rng = np.random.default_rng(seed)
    Dv = shape[-1]
    o = offset + rng.standard_normal(shape)
    gate = rng.standard_normal(shape)
    weight = rng.uniform(0.5, 1.5, Dv).astype(np.float32)
    bias = (0.1 * rng.standard_normal(Dv)).astype(np.float32)
    return dict(o=_cast(o, dtype), gate=_cast(gate, dtype), weight=weight, bias=bias)

