"""MI355X (gfx950) delta-rule sequence mixer: Python binding of libdeltanet.so.

Argument marshalling only.  Every step of the delta rule runs in the HIP kernels
behind the C ABI declared in ``include/deltanet.h``; torch provides device memory
and the stream.  There is no CPU path: without the built library, or without a GPU,
the calls raise.

The rule (frankenstein "DeltaNet Attention" page, module docstring; gate order of
the nnterp "linear_attention" page): per (sequence, value head), with the state S
mapping keys to values and a = exp(g_t),

    S_t = a S_{t-1} - beta_t (a S_{t-1} k_t - v_t) k_t^T,    o_t = scale * S_t q_t.

States are fp32 ``[N, Hv, Dk, Dv]`` holding S^T (key-major).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["chunk_fwd", "chunk_fwd_path", "chunk_bwd", "recurrent_fwd", "recurrent_bwd", "decode_step", "norm_gate", "causal_conv", "conv_qkv",
           "causal_conv_step", "workspace_bytes", "chunk_bwd_workspace_bytes", "lib_path", "load_library",
           "DeltaNetError", "DN_OK", "DN_ERR_INVALID_ARG", "DN_ERR_UNSUPPORTED",
           "DN_ERR_HIP", "DN_ERR_WORKSPACE", "EXPORTED"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdeltanet.so")

DN_OK, DN_ERR_INVALID_ARG, DN_ERR_UNSUPPORTED, DN_ERR_HIP, DN_ERR_WORKSPACE = 0, 1, 2, 3, 4
DN_F32, DN_BF16 = 0, 1
EXPORTED = ("dn_chunk_fwd", "dn_chunk_fwd_workspace_bytes", "dn_decode_step", "dn_decode_step_ex",
            "dn_norm_gate", "dn_recurrent_fwd", "dn_causal_conv", "dn_causal_conv_step",
            "dn_recurrent_bwd", "dn_recurrent_bwd_workspace_bytes", "dn_chunk_fwd_path",
            "dn_chunk_fwd_noalloc", "dn_chunk_bwd", "dn_chunk_bwd_workspace_bytes", "dn_conv_qkv",
            "dn_status_str", "dn_version")


class DeltaNetError(RuntimeError):
    pass


class _Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("Hqk", ctypes.c_int32), ("Hv", ctypes.c_int32), ("Dk", ctypes.c_int32),
                ("Dv", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("scale", ctypes.c_float),
                ("flags", ctypes.c_int32), ("l2norm_eps", ctypes.c_float)]


class _ConvShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("C", ctypes.c_int32), ("width", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("activation", ctypes.c_int32)]


class _QkvSplit(ctypes.Structure):
    _fields_ = [("Hqk", ctypes.c_int32), ("Hv", ctypes.c_int32), ("Dk", ctypes.c_int32),
                ("Dv", ctypes.c_int32), ("qk_l2norm", ctypes.c_int32), ("eps", ctypes.c_float)]


class _Epilogue(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("eps", ctypes.c_float), ("weight", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("gate", ctypes.c_void_p)]


DN_NORM_RMS, DN_NORM_LAYER = 0, 1
_NORM_KINDS = {"rms": DN_NORM_RMS, "layer": DN_NORM_LAYER}

DN_QK_L2NORM = 1
DN_GATE_PER_KEY = 2


def _flags(qk_l2norm: bool, l2norm_eps: float, gate_per_key: bool):
    f = (DN_QK_L2NORM if qk_l2norm else 0) | (DN_GATE_PER_KEY if gate_per_key else 0)
    return f, float(l2norm_eps)


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libdeltanet.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m delta_rule_recurrent_chunked_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        sp = ctypes.POINTER(_Shape)
        lib.dn_chunk_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.dn_chunk_fwd.restype = ctypes.c_int
        lib.dn_chunk_fwd_workspace_bytes.argtypes = [sp]
        lib.dn_chunk_fwd_workspace_bytes.restype = sz
        lib.dn_chunk_fwd_path.argtypes = [sp, sz]
        lib.dn_chunk_fwd_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.dn_chunk_fwd_noalloc.restype = ctypes.c_int
        lib.dn_chunk_fwd_path.restype = ctypes.c_int32
        lib.dn_decode_step.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp]
        ep = ctypes.POINTER(_Epilogue)
        lib.dn_decode_step_ex.argtypes = [sp, vp, vp, vp, vp, vp, vp, ep, vp, vp]
        lib.dn_decode_step_ex.restype = ctypes.c_int
        lib.dn_norm_gate.argtypes = [sp, ep, vp, vp, vp]
        lib.dn_recurrent_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.dn_recurrent_bwd.argtypes = [sp] + [vp] * 17 + [sz, vp]
        lib.dn_recurrent_bwd.restype = ctypes.c_int
        lib.dn_chunk_bwd.argtypes = [sp] + [vp] * 16 + [sz, vp]
        lib.dn_chunk_bwd.restype = ctypes.c_int
        lib.dn_chunk_bwd_workspace_bytes.argtypes = [sp]
        lib.dn_chunk_bwd_workspace_bytes.restype = sz
        lib.dn_recurrent_bwd_workspace_bytes.argtypes = [sp]
        lib.dn_recurrent_bwd_workspace_bytes.restype = sz
        cs = ctypes.POINTER(_ConvShape)
        lib.dn_causal_conv.argtypes = [cs, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.dn_causal_conv.restype = ctypes.c_int
        lib.dn_conv_qkv.argtypes = [cs, ctypes.POINTER(_QkvSplit), vp, vp, vp, vp, vp, vp, vp, vp,
                                    vp, vp]
        lib.dn_conv_qkv.restype = ctypes.c_int
        lib.dn_causal_conv_step.argtypes = [cs, vp, vp, vp, vp, vp, vp]
        lib.dn_causal_conv_step.restype = ctypes.c_int
        lib.dn_recurrent_fwd.restype = ctypes.c_int
        lib.dn_norm_gate.restype = ctypes.c_int
        lib.dn_decode_step.restype = ctypes.c_int
        lib.dn_status_str.argtypes = [ctypes.c_int]
        lib.dn_status_str.restype = ctypes.c_char_p
        lib.dn_version.argtypes = []
        lib.dn_version.restype = ctypes.c_int32
        _lib = lib
    return _lib


def _raise(code: int, what: str):
    msg = f"{what}: {load_library().dn_status_str(code).decode()}"
    if code in (DN_ERR_INVALID_ARG, DN_ERR_WORKSPACE):
        raise ValueError(msg)
    if code == DN_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise DeltaNetError(msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DN_F32
    if t.dtype == torch.bfloat16:
        return DN_BF16
    raise NotImplementedError(f"q/k/v dtype {t.dtype} is not supported (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_bytes(B: int, T: int, Hqk: int, Hv: int, Dk: int, Dv: int, dtype: torch.dtype,
                    num_seqs: Optional[int] = None, chunk_size: int = 64,
                    g_per_key: bool = False, qk_l2norm: bool = False) -> int:
    """Device workspace (bytes) ``dn_chunk_fwd`` needs for these sizes (only the two-kernel
    matrix-core path of a log decay per key channel at d_k = 128 uses one)."""
    s = _Shape(B, T, B if num_seqs is None else num_seqs, Hqk, Hv, Dk, Dv,
               DN_BF16 if dtype == torch.bfloat16 else DN_F32, chunk_size, 1.0,
               *_flags(qk_l2norm, 1e-6, g_per_key))
    return int(load_library().dn_chunk_fwd_workspace_bytes(ctypes.byref(s)))


def chunk_bwd_workspace_bytes(B: int, T: int, Hqk: int, Hv: int, Dk: int, Dv: int,
                              dtype: torch.dtype, num_seqs: Optional[int] = None,
                              qk_l2norm: bool = False) -> int:
    """Device workspace (bytes) ``dn_chunk_bwd`` needs for these sizes (0 where the reverse
    pass does not support them)."""
    s = _Shape(B, T, B if num_seqs is None else num_seqs, Hqk, Hv, Dk, Dv,
               DN_BF16 if dtype == torch.bfloat16 else DN_F32, 64, 1.0, *_flags(qk_l2norm, 1e-6, False))
    return int(load_library().dn_chunk_bwd_workspace_bytes(ctypes.byref(s)))


_PATHS = {-1: "invalid", 0: "fused", 1: "channel_gate_two_kernels", 2: "channel_gate_one_kernel",
          3: "vector"}


def chunk_fwd_path(B: int, T: int, Hqk: int, Hv: int, Dk: int, Dv: int, dtype: torch.dtype,
                   num_seqs: Optional[int] = None, chunk_size: int = 64, g_per_key: bool = False,
                   qk_l2norm: bool = False, workspace_bytes: Optional[int] = None) -> str:
    """Which kernels ``chunk_fwd`` runs for these sizes: "fused" (one matrix-core kernel, bf16
    d = 128 or 64), "channel_gate_two_kernels" / "channel_gate_one_kernel" (per-key-channel
    gates on the matrix cores, with / without enough workspace), "vector" (the vector-ALU
    chunked kernel, about 100x slower), or "invalid".  ``workspace_bytes`` defaults to what
    :func:`chunk_fwd` allocates itself."""
    s = _Shape(B, T, B if num_seqs is None else num_seqs, Hqk, Hv, Dk, Dv,
               DN_BF16 if dtype == torch.bfloat16 else DN_F32, chunk_size, 1.0,
               *_flags(qk_l2norm, 1e-6, g_per_key))
    lib = load_library()
    if workspace_bytes is None:
        workspace_bytes = int(lib.dn_chunk_fwd_workspace_bytes(ctypes.byref(s)))
    return _PATHS[int(lib.dn_chunk_fwd_path(ctypes.byref(s), int(workspace_bytes)))]


def _prompt_args(q, k, v, beta, g, initial_state, output_final_state, cu_seqlens, scale,
                 chunk_size, out, final_state, check_cu_seqlens, qk_l2norm, l2norm_eps):
    """Checks and allocations shared by the whole-sequence calls; returns
    (shape, out, final_state, N)."""
    _dev(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [B, T, Hqk, Dk]")
    B, T, Hqk, Dk = q.shape
    _dev(k, "k", q.dtype, q.shape)
    if v.dim() != 4:
        raise ValueError("v must be [B, T, Hv, Dv]")
    _dev(v, "v", q.dtype)
    Hv, Dv = v.shape[2], v.shape[3]
    if tuple(v.shape[:2]) != (B, T):
        raise ValueError("v must be [B, T, Hv, Dv] with the batch and length of q")
    _dev(beta, "beta", torch.float32, (B, T, Hv))
    per_key = g is not None and g.dim() == 4
    if g is not None:
        _dev(g, "g", torch.float32, (B, T, Hv, Dk) if per_key else (B, T, Hv))
    if cu_seqlens is not None:
        _dev(cu_seqlens, "cu_seqlens", torch.int32)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be [N + 1] with N >= 1")
        N = cu_seqlens.numel() - 1
        if B != 1:
            raise ValueError("a packed batch (cu_seqlens) must have B == 1")
        if check_cu_seqlens:
            c = cu_seqlens.cpu()
            if int(c[0]) != 0 or int(c[-1]) != T or bool((c[1:] < c[:-1]).any()):
                raise ValueError("cu_seqlens must start at 0, not decrease and end at T")
    else:
        N = B
    if initial_state is not None:
        _dev(initial_state, "initial_state", torch.float32, (N, Hv, Dk, Dv))
    dev = q.device
    if out is None:
        out = torch.empty((B, T, Hv, Dv), dtype=q.dtype, device=dev)
    else:
        _dev(out, "out", q.dtype, (B, T, Hv, Dv))
    if final_state is None and output_final_state:
        final_state = torch.empty((N, Hv, Dk, Dv), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _dev(final_state, "final_state", torch.float32, (N, Hv, Dk, Dv))
    shape = _Shape(B, T, N, Hqk, Hv, Dk, Dv, _dtype_code(q), chunk_size, float(scale),
                   *_flags(qk_l2norm, l2norm_eps, per_key))
    return shape, out, final_state, N


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
              g: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
              output_final_state: bool = True, cu_seqlens: Optional[torch.Tensor] = None,
              scale: float = 1.0, chunk_size: int = 64, out: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, check_cu_seqlens: bool = False,
              qk_l2norm: bool = False, l2norm_eps: float = 1e-6
              ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Delta rule over whole sequences (prefill), chunkwise-parallel form.

    q, k ``[B, T, Hqk, Dk]``, v ``[B, T, Hv, Dv]`` (float32 or bfloat16, one dtype);
    beta, g ``[B, T, Hv]`` float32 (g None: plain rule; g ``[B, T, Hv, Dk]``: one log decay
    per key channel); initial_state
    ``[N, Hv, Dk, Dv]`` float32 or None (zero state); cu_seqlens int32 ``[N + 1]``
    packs N sequences along T (B == 1).  Returns ``(o [B, T, Hv, Dv], final_state or
    None)``.  ``final_state`` may be passed (and may be ``initial_state``, to update
    it in place); ``out`` and ``workspace`` may be passed to avoid allocation.
    The kernels trust cu_seqlens (``cu[0] == 0``, non-decreasing, ``cu[N] == T``);
    ``check_cu_seqlens=True`` checks it on a host copy first (a synchronising copy, which
    also cannot be captured in a HIP graph), for debugging.
    ``qk_l2norm`` normalises q and k inside the call, x / sqrt(|x|^2 + l2norm_eps).
    """
    lib = load_library()
    shape, out, final_state, _ = _prompt_args(q, k, v, beta, g, initial_state, output_final_state,
                                              cu_seqlens, scale, chunk_size, out, final_state,
                                              check_cu_seqlens, qk_l2norm, l2norm_eps)
    dev = q.device
    need = int(lib.dn_chunk_fwd_workspace_bytes(ctypes.byref(shape)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if need else None
    else:
        _dev(workspace, "workspace", torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel()
    with torch.cuda.device(dev):
        rc = lib.dn_chunk_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                              _ptr(g), _ptr(initial_state), _ptr(final_state),
                              _ptr(cu_seqlens), _ptr(out), _ptr(workspace), ws_bytes,
                              _stream(dev))
    if rc != DN_OK:
        _raise(rc, "dn_chunk_fwd")
    return out, final_state


def recurrent_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                  g: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
                  output_final_state: bool = True, cu_seqlens: Optional[torch.Tensor] = None,
                  scale: float = 1.0, out: Optional[torch.Tensor] = None,
                  final_state: Optional[torch.Tensor] = None, state_trace: bool = False,
                  check_cu_seqlens: bool = False, qk_l2norm: bool = False,
                  l2norm_eps: float = 1e-6):
    """The rule token by token over whole sequences (the recurrent route), same arguments
    as :func:`chunk_fwd`.  Returns ``(o, final_state, trace)`` where ``trace`` is the
    state after every token, ``[B, T, Hv, Dk, Dv]`` float32, when ``state_trace`` (else
    None)."""
    lib = load_library()
    shape, out, final_state, _ = _prompt_args(q, k, v, beta, g, initial_state, output_final_state,
                                              cu_seqlens, scale, 64, out, final_state,
                                              check_cu_seqlens, qk_l2norm, l2norm_eps)
    B, T, Hv, Dv = out.shape
    Dk = q.shape[3]
    trace = None
    if state_trace:
        trace = torch.empty((B, T, Hv, Dk, Dv), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        rc = lib.dn_recurrent_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                  _ptr(g), _ptr(initial_state), _ptr(final_state),
                                  _ptr(cu_seqlens), _ptr(out), _ptr(trace), _stream(q.device))
    if rc != DN_OK:
        _raise(rc, "dn_recurrent_fwd")
    return out, final_state, trace


def recurrent_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                  g: Optional[torch.Tensor], initial_state: Optional[torch.Tensor],
                  state_trace: torch.Tensor, d_o: torch.Tensor,
                  d_final_state: Optional[torch.Tensor] = None,
                  cu_seqlens: Optional[torch.Tensor] = None, scale: float = 1.0,
                  qk_l2norm: bool = False, l2norm_eps: float = 1e-6,
                  check_cu_seqlens: bool = False) -> dict:
    """Reverse pass of the rule: gradients of a loss with dL/do = ``d_o`` and dL/d final
    state = ``d_final_state`` for q, k, v, beta, g and the initial state, from the state
    trace that :func:`recurrent_fwd` returned for the same inputs (``state_trace=True``).
    One gate per head (g ``[B, T, Hv]``), one per key channel (g ``[B, T, Hv, Dk]``) or
    none.  With ``qk_l2norm`` (as given to the forward call) dq and dk are the gradients for
    the raw q and k.  Returns a dict of float32 tensors dq, dk (``[B, T, Hqk, Dk]``), dv,
    dbeta, dg (g's shape; None without g) and d_initial_state."""
    lib = load_library()
    shape, _, _, N = _prompt_args(q, k, v, beta, g, initial_state, False, cu_seqlens, scale, 64,
                                  None, None, check_cu_seqlens, qk_l2norm, l2norm_eps)
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    _dev(state_trace, "state_trace", torch.float32, (B, T, Hv, Dk, Dv))
    _dev(d_o, "d_o", q.dtype, (B, T, Hv, Dv))
    if d_final_state is not None:
        _dev(d_final_state, "d_final_state", torch.float32, (N, Hv, Dk, Dv))
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dq=torch.empty((B, T, Hqk, Dk), **f32), dk=torch.empty((B, T, Hqk, Dk), **f32),
               dv=torch.empty((B, T, Hv, Dv), **f32), dbeta=torch.empty((B, T, Hv), **f32),
               dg=torch.empty(tuple(g.shape), **f32) if g is not None else None,
               d_initial_state=torch.empty((N, Hv, Dk, Dv), **f32))
    need = int(lib.dn_recurrent_bwd_workspace_bytes(ctypes.byref(shape)))
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    with torch.cuda.device(dev):
        rc = lib.dn_recurrent_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                  _ptr(g), _ptr(initial_state), _ptr(state_trace), _ptr(d_o),
                                  _ptr(d_final_state), _ptr(cu_seqlens), _ptr(out["dq"]),
                                  _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]),
                                  _ptr(out["dg"]), _ptr(out["d_initial_state"]), _ptr(ws), need,
                                  _stream(dev))
    if rc != DN_OK:
        _raise(rc, "dn_recurrent_bwd")
    return out


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
              g: Optional[torch.Tensor], initial_state: Optional[torch.Tensor], d_o: torch.Tensor,
              d_final_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, scale: float = 1.0,
              workspace: Optional[torch.Tensor] = None, qk_l2norm: bool = False,
              l2norm_eps: float = 1e-6) -> dict:
    """Reverse pass of the chunked form (no state trace): gradients of a loss with dL/do =
    ``d_o`` and dL/d final state = ``d_final_state`` for q, k, v, beta, g and the initial
    state.  bf16, Dk = Dv = 128, one gate per head or none; with ``qk_l2norm`` the rule
    reads q and k normalised inside the call (as ``chunk_fwd(..., qk_l2norm=True)``) and
    dq, dk are the gradients for the raw q and k.  Returns a dict of float32 tensors dq, dk
    (``[B, T, Hqk, Dk]``), dv, dbeta, dg (None without g) and d_initial_state.
    ``workspace`` (uint8, at least the size the library asks for) may be passed to avoid
    its allocation."""
    lib = load_library()
    shape, _, _, N = _prompt_args(q, k, v, beta, g, initial_state, False, cu_seqlens, scale, 64,
                                  None, None, False, qk_l2norm, l2norm_eps)
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    _dev(d_o, "d_o", q.dtype, (B, T, Hv, Dv))
    if d_final_state is not None:
        _dev(d_final_state, "d_final_state", torch.float32, (N, Hv, Dk, Dv))
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dq=torch.empty((B, T, Hqk, Dk), **f32), dk=torch.empty((B, T, Hqk, Dk), **f32),
               dv=torch.empty((B, T, Hv, Dv), **f32), dbeta=torch.empty((B, T, Hv), **f32),
               dg=torch.empty((B, T, Hv), **f32) if g is not None else None,
               d_initial_state=torch.empty((N, Hv, Dk, Dv), **f32))
    need = int(lib.dn_chunk_bwd_workspace_bytes(ctypes.byref(shape)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _dev(workspace, "workspace", torch.uint8)
    with torch.cuda.device(dev):
        rc = lib.dn_chunk_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                              _ptr(initial_state), _ptr(d_o), _ptr(d_final_state), _ptr(cu_seqlens),
                              _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]),
                              _ptr(out["dg"]), _ptr(out["d_initial_state"]), _ptr(workspace),
                              workspace.numel(), _stream(dev))
    if rc != DN_OK:
        _raise(rc, "dn_chunk_bwd")
    return out


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                g: Optional[torch.Tensor], state: torch.Tensor, scale: float = 1.0,
                out: Optional[torch.Tensor] = None, qk_l2norm: bool = False,
                l2norm_eps: float = 1e-6, norm: Optional[str] = None, norm_eps: float = 1e-6,
                norm_weight: Optional[torch.Tensor] = None,
                norm_bias: Optional[torch.Tensor] = None,
                out_gate: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One token per sequence against the cached ``state`` (updated in place).

    q, k ``[N, Hqk, Dk]``, v ``[N, Hv, Dv]``; beta, g ``[N, Hv]`` float32 (g may be
    None, or ``[N, Hv, Dk]``: one log decay per key channel); state ``[N, Hv, Dk, Dv]``
    float32.  Returns o ``[N, Hv, Dv]``.
    ``qk_l2norm`` normalises q and k inside the call, as in :func:`chunk_fwd`.
    ``norm`` ("rms" or "layer") fuses the readout epilogue of :func:`norm_gate` (with
    ``norm_eps``, ``norm_weight``, ``norm_bias`` and the output gate ``out_gate``, shaped
    like o): ``out`` then holds the epilogue's result.
    """
    lib = load_library()
    _dev(q, "q")
    if q.dim() != 3:
        raise ValueError("q must be [N, Hqk, Dk]")
    N, Hqk, Dk = q.shape
    _dev(k, "k", q.dtype, q.shape)
    _dev(v, "v", q.dtype)
    if v.dim() != 3 or v.shape[0] != N:
        raise ValueError("v must be [N, Hv, Dv]")
    Hv, Dv = v.shape[1], v.shape[2]
    _dev(beta, "beta", torch.float32, (N, Hv))
    per_key = g is not None and g.dim() == 3
    if g is not None:
        _dev(g, "g", torch.float32, (N, Hv, Dk) if per_key else (N, Hv))
    _dev(state, "state", torch.float32, (N, Hv, Dk, Dv))
    if out is None:
        out = torch.empty((N, Hv, Dv), dtype=q.dtype, device=q.device)
    else:
        _dev(out, "out", q.dtype, (N, Hv, Dv))
    shape = _Shape(N, 1, N, Hqk, Hv, Dk, Dv, _dtype_code(q), 0, float(scale),
                   *_flags(qk_l2norm, l2norm_eps, per_key))
    ep = None
    if norm is not None:
        ep = _epilogue(norm, norm_eps, norm_weight, norm_bias, out_gate, Dv, q.dtype, (N, Hv, Dv))
    with torch.cuda.device(q.device):
        rc = lib.dn_decode_step_ex(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                   _ptr(g), _ptr(state), None if ep is None else ctypes.byref(ep),
                                   _ptr(out), _stream(q.device))
    if rc != DN_OK:
        _raise(rc, "dn_decode_step_ex")
    return out


def _epilogue(kind, eps, weight, bias, gate, Dv, dtype, shape) -> _Epilogue:
    if kind not in _NORM_KINDS:
        raise ValueError(f"norm must be one of {sorted(_NORM_KINDS)}")
    if weight is not None:
        _dev(weight, "norm_weight", torch.float32, (Dv,))
    if bias is not None:
        _dev(bias, "norm_bias", torch.float32, (Dv,))
    if gate is not None:
        _dev(gate, "out_gate", dtype, shape)
    return _Epilogue(_NORM_KINDS[kind], float(eps), _ptr(weight), _ptr(bias), _ptr(gate))


def norm_gate(o: torch.Tensor, norm: str = "rms", eps: float = 1e-6,
              weight: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
              gate: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None
              ) -> torch.Tensor:
    """Readout epilogue over a prefill's output o ``[B, T, Hv, Dv]``: per (token, head)
    an RMS ("rms") or layer ("layer") normalisation over Dv with ``weight`` (and
    ``bias``, layer only) of length Dv, then ``* silu(gate)`` when ``gate`` (shaped like
    o) is given.  ``out`` may be ``o`` (in place)."""
    lib = load_library()
    _dev(o, "o")
    if o.dim() != 4:
        raise ValueError("o must be [B, T, Hv, Dv]")
    B, T, Hv, Dv = o.shape
    if out is None:
        out = torch.empty_like(o)
    else:
        _dev(out, "out", o.dtype, tuple(o.shape))
    ep = _epilogue(norm, eps, weight, bias, gate, Dv, o.dtype, tuple(o.shape))
    shape = _Shape(B, T, B, Hv, Hv, Dv, Dv, _dtype_code(o), 0, 1.0, 0, 0.0)
    with torch.cuda.device(o.device):
        rc = lib.dn_norm_gate(ctypes.byref(shape), ctypes.byref(ep), _ptr(o), _ptr(out),
                              _stream(o.device))
    if rc != DN_OK:
        _raise(rc, "dn_norm_gate")
    return out


_ACTIVATIONS = {None: 0, "none": 0, "silu": 1}


def causal_conv(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                initial_state: Optional[torch.Tensor] = None, output_final_state: bool = True,
                cu_seqlens: Optional[torch.Tensor] = None, activation: Optional[str] = "silu",
                out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None
                ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Short causal depthwise convolution (+ silu) over whole sequences.

    x ``[B, T, C]`` (float32 or bfloat16; C a multiple of 8); weight ``[C, W]`` float32
    (W in 2..8, the last tap on the current token); bias ``[C]`` float32; initial_state
    ``[N, C, W - 1]`` in x's dtype (the W - 1 inputs before each sequence, oldest first)
    or None (zeros); cu_seqlens int32 ``[N + 1]`` packs N sequences (B == 1).  Returns
    ``(y [B, T, C], final_state [N, C, W - 1] or None)``."""
    lib = load_library()
    _dev(x, "x")
    if x.dim() != 3:
        raise ValueError("x must be [B, T, C]")
    B, T, C = x.shape
    _dev(weight, "weight", torch.float32)
    if weight.dim() != 2 or weight.shape[0] != C:
        raise ValueError("weight must be [C, W]")
    W = weight.shape[1]
    if bias is not None:
        _dev(bias, "bias", torch.float32, (C,))
    if cu_seqlens is not None:
        _dev(cu_seqlens, "cu_seqlens", torch.int32)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _dev(initial_state, "initial_state", x.dtype, (N, C, W - 1))
    if out is None:
        out = torch.empty_like(x)
    else:
        _dev(out, "out", x.dtype, (B, T, C))
    if final_state is None and output_final_state:
        final_state = torch.empty((N, C, W - 1), dtype=x.dtype, device=x.device)
    elif final_state is not None:
        _dev(final_state, "final_state", x.dtype, (N, C, W - 1))
    if activation not in _ACTIVATIONS:
        raise ValueError("activation must be 'silu' or None")
    shape = _ConvShape(B, T, N, C, W, _dtype_code(x), _ACTIVATIONS[activation])
    with torch.cuda.device(x.device):
        rc = lib.dn_causal_conv(ctypes.byref(shape), _ptr(x), _ptr(weight), _ptr(bias),
                                _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), _ptr(out),
                                _stream(x.device))
    if rc != DN_OK:
        _raise(rc, "dn_causal_conv")
    return out, final_state


def conv_qkv(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor], Hqk: int, Hv: int,
             Dk: int, Dv: int, initial_state: Optional[torch.Tensor] = None,
             output_final_state: bool = True, cu_seqlens: Optional[torch.Tensor] = None,
             activation: Optional[str] = "silu", qk_l2norm: bool = True, eps: float = 1e-6
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """The prologue in front of the rule in one pass: :func:`causal_conv` over
    x = [q | k | v] projections ``[B, T, 2 Hqk Dk + Hv Dv]``, split into q, k
    ``[B, T, Hqk, Dk]`` and v ``[B, T, Hv, Dv]`` with q and k L2-normalised per head
    (``qk_l2norm``, x / sqrt(|x|^2 + eps)).  Returns ``(q, k, v, final_state)``; hand q, k, v
    to :func:`chunk_fwd` without ``qk_l2norm``."""
    lib = load_library()
    _dev(x, "x")
    if x.dim() != 3:
        raise ValueError("x must be [B, T, C]")
    B, T, C = x.shape
    _dev(weight, "weight", torch.float32)
    if weight.dim() != 2 or weight.shape[0] != C:
        raise ValueError("weight must be [C, W]")
    W = weight.shape[1]
    if bias is not None:
        _dev(bias, "bias", torch.float32, (C,))
    if cu_seqlens is not None:
        _dev(cu_seqlens, "cu_seqlens", torch.int32)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _dev(initial_state, "initial_state", x.dtype, (N, C, W - 1))
    final_state = torch.empty((N, C, W - 1), dtype=x.dtype, device=x.device) if output_final_state else None
    if activation not in _ACTIVATIONS:
        raise ValueError("activation must be 'silu' or None")
    q = torch.empty((B, T, Hqk, Dk), dtype=x.dtype, device=x.device)
    k = torch.empty((B, T, Hqk, Dk), dtype=x.dtype, device=x.device)
    v = torch.empty((B, T, Hv, Dv), dtype=x.dtype, device=x.device)
    shape = _ConvShape(B, T, N, C, W, _dtype_code(x), _ACTIVATIONS[activation])
    split = _QkvSplit(Hqk, Hv, Dk, Dv, int(bool(qk_l2norm)), float(eps))
    with torch.cuda.device(x.device):
        rc = lib.dn_conv_qkv(ctypes.byref(shape), ctypes.byref(split), _ptr(x), _ptr(weight),
                             _ptr(bias), _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens),
                             _ptr(q), _ptr(k), _ptr(v), _stream(x.device))
    if rc != DN_OK:
        _raise(rc, "dn_conv_qkv")
    return q, k, v, final_state


def causal_conv_step(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor],
                     conv_state: torch.Tensor, activation: Optional[str] = "silu",
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One token per sequence: x ``[N, C]``, conv_state ``[N, C, W - 1]`` (x's dtype)
    updated in place.  Returns y ``[N, C]``."""
    lib = load_library()
    _dev(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [N, C]")
    N, C = x.shape
    _dev(weight, "weight", torch.float32)
    if weight.dim() != 2 or weight.shape[0] != C:
        raise ValueError("weight must be [C, W]")
    W = weight.shape[1]
    if bias is not None:
        _dev(bias, "bias", torch.float32, (C,))
    _dev(conv_state, "conv_state", x.dtype, (N, C, W - 1))
    if out is None:
        out = torch.empty_like(x)
    else:
        _dev(out, "out", x.dtype, (N, C))
    if activation not in _ACTIVATIONS:
        raise ValueError("activation must be 'silu' or None")
    shape = _ConvShape(N, 1, N, C, W, _dtype_code(x), _ACTIVATIONS[activation])
    with torch.cuda.device(x.device):
        rc = lib.dn_causal_conv_step(ctypes.byref(shape), _ptr(x), _ptr(weight), _ptr(bias),
                                     _ptr(conv_state), _ptr(out), _stream(x.device))
    if rc != DN_OK:
        _raise(rc, "dn_causal_conv_step")
    return out

