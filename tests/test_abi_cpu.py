"""The C-ABI library on a machine without a GPU: it loads, exports every entry point the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import delta_rule_recurrent_chunked_amd as dn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "deltanet.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dn_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = dn.load_library()
    declared = _declared()
    assert set(declared) == set(dn.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.dn_version() >= 10000


def test_status_strings():
    lib = dn.load_library()
    for code in range(5):
        assert lib.dn_status_str(code)
    assert b"invalid" in lib.dn_status_str(dn.DN_ERR_INVALID_ARG)


def _shape(**kw):
    d = dict(B=1, T=64, num_seqs=1, Hqk=2, Hv=2, Dk=16, Dv=16, dtype=dn.DN_BF16, chunk_size=64,
             scale=1.0)
    d.update(kw)
    return dn._Shape(**d)


def _chunk(shape, ptr=16, **over):
    lib = dn.load_library()
    p = ctypes.c_void_p(ptr)
    args = dict(q=p, k=p, v=p, beta=p, g=None, h0=None, hT=None, cu=None, o=p, ws=None, wsb=0)
    args.update(over)
    return lib.dn_chunk_fwd(ctypes.byref(shape), args["q"], args["k"], args["v"], args["beta"],
                            args["g"], args["h0"], args["hT"], args["cu"], args["o"], args["ws"],
                            args["wsb"], None)


@pytest.mark.parametrize("bad,code", [
    (dict(Hqk=3, Hv=4), dn.DN_ERR_INVALID_ARG),        # Hv not a multiple of Hqk
    (dict(Hqk=0), dn.DN_ERR_INVALID_ARG),
    (dict(T=-1), dn.DN_ERR_INVALID_ARG),
    (dict(B=2, num_seqs=1), dn.DN_ERR_INVALID_ARG),     # num_seqs != B without cu_seqlens
    (dict(Dk=48), dn.DN_ERR_UNSUPPORTED),
    (dict(Dv=256), dn.DN_ERR_UNSUPPORTED),
    (dict(chunk_size=128), dn.DN_ERR_UNSUPPORTED),
    (dict(dtype=7), dn.DN_ERR_UNSUPPORTED),
    (dict(flags=4), dn.DN_ERR_INVALID_ARG),             # unknown flag bit
    (dict(flags=2), dn.DN_ERR_INVALID_ARG),             # gates per key channel without g
    (dict(flags=1, l2norm_eps=-1e-6), dn.DN_ERR_INVALID_ARG),
    (dict(flags=1, l2norm_eps=float("inf")), dn.DN_ERR_INVALID_ARG),
    (dict(flags=1, l2norm_eps=float("nan")), dn.DN_ERR_INVALID_ARG),
])
def test_chunk_fwd_rejects_bad_shapes(bad, code):
    assert _chunk(_shape(**bad)) == code


def test_chunk_fwd_rejects_null_and_misaligned():
    assert _chunk(_shape(), q=None) == dn.DN_ERR_INVALID_ARG
    assert _chunk(_shape(), ptr=18) == dn.DN_ERR_INVALID_ARG
    # packed batch needs B == 1
    assert _chunk(_shape(B=2, num_seqs=3), cu=ctypes.c_void_p(16)) == dn.DN_ERR_INVALID_ARG


def test_decode_rejects_bad_shapes():
    lib = dn.load_library()
    p = ctypes.c_void_p(16)
    s = _shape(B=4, T=2, num_seqs=4)
    assert lib.dn_decode_step(ctypes.byref(s), p, p, p, p, None, p, p, None) == dn.DN_ERR_INVALID_ARG
    s = _shape(B=4, T=1, num_seqs=4, Dk=24)
    assert lib.dn_decode_step(ctypes.byref(s), p, p, p, p, None, p, p, None) == dn.DN_ERR_UNSUPPORTED
    s = _shape(B=4, T=1, num_seqs=4)
    assert lib.dn_decode_step(ctypes.byref(s), p, None, p, p, None, p, p, None) == dn.DN_ERR_INVALID_ARG
    s = _shape(B=4, T=1, num_seqs=4, flags=4)
    assert lib.dn_decode_step(ctypes.byref(s), p, p, p, p, None, p, p, None) == dn.DN_ERR_INVALID_ARG
    s = _shape(B=4, T=1, num_seqs=4, flags=1, l2norm_eps=-1.0)
    assert lib.dn_decode_step(ctypes.byref(s), p, p, p, p, None, p, p, None) == dn.DN_ERR_INVALID_ARG


def test_workspace_query_is_host_only():
    import torch
    assert dn.workspace_bytes(1, 64, 2, 2, 16, 16, torch.float32) == 0


def test_python_wrapper_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        dn.chunk_fwd(q, q, q, torch.zeros(1, 4, 1))


def _ep(**kw):
    d = dict(kind=dn.DN_NORM_RMS, eps=1e-6, weight=None, bias=None, gate=None)
    d.update(kw)
    return dn._Epilogue(**d)


@pytest.mark.parametrize("bad", [
    dict(kind=2),                                   # unknown norm
    dict(eps=-1.0),
    dict(eps=float("nan")),
    dict(bias=16),                                  # a bias with the RMS norm
    dict(kind=dn.DN_NORM_LAYER, gate=24),           # misaligned gate
    dict(kind=dn.DN_NORM_LAYER, weight=18),         # misaligned weight
])
def test_epilogue_rejects_bad_specs(bad):
    lib = dn.load_library()
    p = ctypes.c_void_p(16)
    ep = _ep(**bad)
    s = _shape(B=4, T=1, num_seqs=4)
    assert lib.dn_decode_step_ex(ctypes.byref(s), p, p, p, p, None, p, ctypes.byref(ep), p,
                                 None) == dn.DN_ERR_INVALID_ARG
    s = _shape(B=2, T=8, num_seqs=2)
    assert lib.dn_norm_gate(ctypes.byref(s), ctypes.byref(ep), p, p, None) == dn.DN_ERR_INVALID_ARG


def test_norm_gate_needs_an_epilogue_and_buffers():
    lib = dn.load_library()
    p = ctypes.c_void_p(16)
    s = _shape(B=2, T=8, num_seqs=2)
    assert lib.dn_norm_gate(ctypes.byref(s), None, p, p, None) == dn.DN_ERR_INVALID_ARG
    ep = _ep(kind=dn.DN_NORM_LAYER)
    assert lib.dn_norm_gate(ctypes.byref(s), ctypes.byref(ep), None, p, None) == dn.DN_ERR_INVALID_ARG
    assert lib.dn_norm_gate(ctypes.byref(s), ctypes.byref(ep), ctypes.c_void_p(20), p, None) == dn.DN_ERR_INVALID_ARG
    s = _shape(B=2, T=8, num_seqs=2, Dv=48)
    assert lib.dn_norm_gate(ctypes.byref(s), ctypes.byref(ep), p, p, None) == dn.DN_ERR_UNSUPPORTED


def _cshape(**kw):
    d = dict(B=1, T=64, num_seqs=1, C=64, width=4, dtype=dn.DN_BF16, activation=1)
    d.update(kw)
    return dn._ConvShape(**d)


@pytest.mark.parametrize("bad,code", [
    (dict(C=60), dn.DN_ERR_INVALID_ARG),                # not a multiple of 8
    (dict(width=1), dn.DN_ERR_UNSUPPORTED),
    (dict(width=9), dn.DN_ERR_UNSUPPORTED),
    (dict(activation=2), dn.DN_ERR_INVALID_ARG),
    (dict(dtype=5), dn.DN_ERR_UNSUPPORTED),
    (dict(B=2, num_seqs=3), dn.DN_ERR_INVALID_ARG),
])
def test_causal_conv_rejects_bad_shapes(bad, code):
    lib = dn.load_library()
    p = ctypes.c_void_p(16)
    s = _cshape(**bad)
    assert lib.dn_causal_conv(ctypes.byref(s), p, p, None, None, None, None, ctypes.c_void_p(32), None) == code


def test_causal_conv_rejects_aliasing_and_misalignment():
    lib = dn.load_library()
    p, q = ctypes.c_void_p(16), ctypes.c_void_p(32)
    s = _cshape()
    assert lib.dn_causal_conv(ctypes.byref(s), p, p, None, None, None, None, p, None) == dn.DN_ERR_INVALID_ARG
    assert lib.dn_causal_conv(ctypes.byref(s), p, p, None, q, q, None, ctypes.c_void_p(48), None) == dn.DN_ERR_INVALID_ARG
    assert lib.dn_causal_conv(ctypes.byref(s), ctypes.c_void_p(24), p, None, None, None, None, q, None) == dn.DN_ERR_INVALID_ARG
    s = _cshape(B=4, T=2, num_seqs=4)
    assert lib.dn_causal_conv_step(ctypes.byref(s), p, p, None, p, q, None) == dn.DN_ERR_INVALID_ARG



@pytest.mark.parametrize("split,code", [
    ((2, 2, 64, 64), dn.DN_ERR_INVALID_ARG),            # 2*2*64 + 2*64 = 384 != C
    ((1, 1, 24, 16), dn.DN_ERR_UNSUPPORTED),            # Dk outside {16, 32, 64, 128}
    ((1, 1, 16, 12), dn.DN_ERR_INVALID_ARG),            # Dv not a multiple of 8
    ((0, 2, 16, 16), dn.DN_ERR_INVALID_ARG),            # no q/k heads
])
def test_conv_qkv_rejects_bad_splits(split, code):
    """dn_conv_qkv's host checks: the split must add up to C, with supported head sizes."""
    lib = dn.load_library()
    p = ctypes.c_void_p(16)
    s = _cshape(C=64)
    sp = dn._QkvSplit(*split, 1, 1e-6)
    assert lib.dn_conv_qkv(ctypes.byref(s), ctypes.byref(sp), p, p, None, None, None, None,
                           ctypes.c_void_p(32), ctypes.c_void_p(48), ctypes.c_void_p(64), None) == code


def test_conv_qkv_rejects_aliasing_eps_and_misalignment():
    lib = dn.load_library()
    p, a, b, c = (ctypes.c_void_p(v) for v in (16, 32, 48, 64))
    s = _cshape(C=64)                                    # 2 * 1 * 16 + 2 * 16
    ok = dn._QkvSplit(1, 2, 16, 16, 1, 1e-6)
    args = lambda q, k, v: (ctypes.byref(s), ctypes.byref(ok), p, p, None, None, None, None, q, k, v, None)
    assert lib.dn_conv_qkv(*args(p, b, c)) == dn.DN_ERR_INVALID_ARG          # q aliases x
    assert lib.dn_conv_qkv(*args(a, a, c)) == dn.DN_ERR_INVALID_ARG          # q aliases k
    assert lib.dn_conv_qkv(*args(ctypes.c_void_p(40), b, c)) == dn.DN_ERR_INVALID_ARG   # misaligned
    for eps in (-1.0, float("inf"), float("nan")):
        bad = dn._QkvSplit(1, 2, 16, 16, 1, eps)
        assert lib.dn_conv_qkv(ctypes.byref(s), ctypes.byref(bad), p, p, None, None, None, None,
                               a, b, c, None) == dn.DN_ERR_INVALID_ARG
    assert lib.dn_conv_qkv(ctypes.byref(s), None, p, p, None, None, None, None, a, b, c, None) == dn.DN_ERR_INVALID_ARG


def test_reverse_pass_host_checks():
    """dn_recurrent_bwd: a decay per key channel needs g, and the workspace query counts Dk
    floats of dg per token and head with that flag."""
    lib = dn.load_library()
    p = ctypes.c_void_p(16)
    args = [p] * 6 + [p, p, None, None] + [p] * 6 + [p, 1 << 30, None]
    s = _shape(B=1, T=8, num_seqs=1, flags=2)
    a2 = list(args)
    a2[4] = None          # g
    assert lib.dn_recurrent_bwd(ctypes.byref(s), *a2) == dn.DN_ERR_INVALID_ARG
    plain = _shape(B=2, T=8, num_seqs=2, Dk=64, Dv=64)
    chg = _shape(B=2, T=8, num_seqs=2, Dk=64, Dv=64, flags=2)
    slices, per_tok = 8, 2 * 8 * plain.Hv   # 8-column slices
    assert lib.dn_recurrent_bwd_workspace_bytes(ctypes.byref(plain)) == slices * per_tok * (2 * 64 + 2) * 4
    assert lib.dn_recurrent_bwd_workspace_bytes(ctypes.byref(chg)) == slices * per_tok * (3 * 64 + 1) * 4


def test_channel_gate_prompt_workspace_query():
    """dn_chunk_fwd_workspace_bytes: 68,352 bytes per (chunk, value head) for a bf16 Dk = 128
    prompt with a log decay per key channel, over a chunk bound that holds for rows and for
    packed sequences; zero for every shape that runs without one."""
    import torch
    rec = 68352
    # a batch of rows: exactly B * ceil(T / 64) chunks
    assert dn.workspace_bytes(4, 2048, 16, 16, 128, 128, torch.bfloat16, g_per_key=True) == 4 * 32 * 16 * rec
    # packed: 5 sequences in 300 tokens -> at most (300 + 63 * 5) // 64 + 1 = 10 chunks
    assert dn.workspace_bytes(1, 300, 2, 4, 128, 128, torch.bfloat16, num_seqs=5, g_per_key=True) == 10 * 4 * rec
    assert dn.workspace_bytes(4, 2048, 16, 16, 128, 128, torch.bfloat16) == 0
    assert dn.workspace_bytes(4, 2048, 16, 16, 128, 128, torch.float32, g_per_key=True) == 0
    assert dn.workspace_bytes(4, 2048, 16, 16, 64, 64, torch.bfloat16, g_per_key=True) == 0
    assert dn.workspace_bytes(4, 2048, 16, 16, 128, 128, torch.bfloat16, chunk_size=32, g_per_key=True) == 0


def test_chunk_fwd_path_reports_the_kernels():
    """The host-only query names the kernels a prompt call runs (the vector-ALU fallback
    included), without touching a device."""
    bf, f32 = torch_dtypes()
    path = dn.chunk_fwd_path
    assert path(4, 2048, 16, 16, 128, 128, bf) == "fused"
    assert path(1, 32768, 32, 32, 128, 128, bf, num_seqs=8) == "fused"
    assert path(4, 2048, 16, 16, 128, 128, bf, qk_l2norm=True) == "fused"
    assert path(4, 2048, 16, 16, 64, 64, bf) == "fused"
    assert path(4, 2048, 16, 16, 64, 64, bf, workspace_bytes=0) == "fused"
    assert path(4, 2048, 16, 16, 64, 64, bf, qk_l2norm=True) == "fused"
    assert path(4, 2048, 16, 16, 64, 64, f32) == "vector"
    assert path(4, 2048, 16, 16, 64, 128, bf) == "vector"
    assert path(4, 2048, 16, 16, 128, 128, f32) == "vector"
    assert path(4, 2048, 16, 16, 128, 128, bf, chunk_size=32) == "vector"
    assert path(4, 2048, 16, 16, 128, 128, bf, g_per_key=True) == "channel_gate_two_kernels"
    assert path(4, 2048, 16, 16, 128, 128, bf, g_per_key=True, workspace_bytes=0) == \
        "channel_gate_one_kernel"
    assert path(4, 2048, 16, 16, 64, 64, bf, g_per_key=True) == "vector"
    assert path(4, 2048, 3, 16, 128, 128, bf) == "invalid"
    assert path(4, 2048, 16, 16, 48, 128, bf) == "invalid"


def test_d64_prompt_workspace_query():
    """dn_chunk_fwd_workspace_bytes is zero for the bf16 d = 64 prompt (one kernel, every
    intermediate on chip), with or without the in-rule normalisation, and for the shapes that
    run on the vector ALUs."""
    import torch
    bf = torch.bfloat16
    assert dn.workspace_bytes(4, 2048, 16, 16, 64, 64, bf) == 0
    assert dn.workspace_bytes(1, 300, 2, 4, 64, 64, bf, num_seqs=5) == 0
    assert dn.workspace_bytes(4, 2048, 16, 16, 64, 64, bf, qk_l2norm=True) == 0
    assert dn.workspace_bytes(4, 2048, 16, 16, 64, 64, torch.float32) == 0
    assert dn.workspace_bytes(4, 2048, 16, 16, 64, 64, bf, chunk_size=32) == 0
    assert dn.workspace_bytes(4, 2048, 16, 16, 64, 32, bf) == 0


def torch_dtypes():
    import torch
    return torch.bfloat16, torch.float32


def test_chunk_fwd_noalloc_rejects_oversized_scratch_on_the_host():
    """The allocation-free prompt call refuses, before any HIP call, a channel-gate prompt
    whose records exceed the static scratch (B4 H16 T2048: 2,048 records of 68,352 B
    against 64 MiB), and checks shapes as dn_chunk_fwd does."""
    lib = dn.load_library()
    p = ctypes.c_void_p(16)
    big = _shape(B=4, T=2048, num_seqs=4, Hqk=16, Hv=16, Dk=128, Dv=128, flags=dn.DN_GATE_PER_KEY)
    assert lib.dn_chunk_fwd_noalloc(ctypes.byref(big), p, p, p, p, p, None, None, None, p,
                                    None) == dn.DN_ERR_WORKSPACE
    assert lib.dn_chunk_fwd_noalloc(ctypes.byref(_shape(Dk=48)), p, p, p, p, None, None, None,
                                    None, p, None) == dn.DN_ERR_UNSUPPORTED
    assert lib.dn_chunk_fwd_noalloc(None, p, p, p, p, None, None, None, None, p,
                                    None) == dn.DN_ERR_INVALID_ARG


def test_chunk_bwd_workspace_query():
    """dn_chunk_bwd_workspace_bytes: per (chunk, value head) the chunk-start state and dL/dM
    (fp32, 2 x 128 x 128 x 4 B) and T, P (bf16, 2 x 64 x 64 x 2 B), over the chunk bound;
    with DN_QK_L2NORM also the normalised q and k (bf16, 2 x tokens x Hqk x 128 x 2 B) and the
    inverse norms of their rows (fp32, 2 x tokens x Hqk x 4 B, rounded up to 256 B); zero for
    shapes the reverse pass does not take."""
    import torch
    bf = torch.bfloat16
    rec = 2 * 128 * 128 * 4 + 2 * 64 * 64 * 2
    assert dn.chunk_bwd_workspace_bytes(4, 2048, 16, 16, 128, 128, bf) == 4 * 32 * 16 * rec
    assert dn.chunk_bwd_workspace_bytes(4, 2048, 16, 16, 128, 128, bf, qk_l2norm=True) == \
        4 * 32 * 16 * rec + 2 * 4 * 2048 * 16 * 128 * 2 + 2 * 4 * 2048 * 16 * 4
    # 3 x 100 x 2 rows of norms = 2400 B -> 2560 B
    assert dn.chunk_bwd_workspace_bytes(1, 100, 3, 3, 128, 128, bf, qk_l2norm=True) == \
        dn.chunk_bwd_workspace_bytes(1, 100, 3, 3, 128, 128, bf) + 2 * 100 * 3 * 128 * 2 + 2560
    assert dn.chunk_bwd_workspace_bytes(4, 2048, 16, 16, 64, 64, bf) == 0
    assert dn.chunk_bwd_workspace_bytes(4, 2048, 16, 16, 128, 128, torch.float32) == 0
