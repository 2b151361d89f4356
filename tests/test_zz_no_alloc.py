"""The allocation-free prompt call (dn_chunk_fwd_noalloc) against dn_chunk_fwd with a
caller-allocated workspace, through the C ABI (needs an MI355X): two calls in a row on one
GPU, the second with a smaller input, each bit for bit equal to the workspace call and
within the bf16 bar of the fp64 oracle, whole tensors and per (sequence, head)."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import delta_rule_recurrent_chunked_amd as dn
from synth import make_case
from tests.gpu_util import host, per_unit_rel, rel_l2, run_oracle, to_inputs, tol

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(x, d):
    lib = dn.load_library()
    o = torch.empty((x.B, x.T, x.Hv, x.Dv), dtype=torch.bfloat16, device="cuda")
    s = torch.empty((x.num_seqs, x.Hv, x.Dk, x.Dv), dtype=torch.float32, device="cuda")
    shape = dn._Shape(x.B, x.T, x.num_seqs, x.Hqk, x.Hv, x.Dk, x.Dv, dn.DN_BF16, 64, 1.0,
                      dn.DN_GATE_PER_KEY if x.g is not None and x.g.ndim == 4 else 0, 1e-6)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.dn_chunk_fwd_noalloc(ctypes.byref(shape), _ptr(d["q"]), _ptr(d["k"]), _ptr(d["v"]),
                                  _ptr(d["beta"]), _ptr(d["g"]), _ptr(d["init"]), _ptr(s),
                                  _ptr(d["cu"]), _ptr(o), stream)
    assert rc == dn.DN_OK, rc
    return o, s


def test_noalloc_matches_workspace_call_twice():
    cases = [
        # first call: 4 heads, two packed sequences (11 + 5 + ... records)
        make_case(B=1, Hqk=2, Hv=4, Dk=128, dtype="bf16", seqlens=[700, 333], g_scale=0.1,
                  init_std=0.02, beta_scale=2.0, seed=71, name="noalloc_first", g_per_key=True),
        # second call, smaller: 2 heads, one 150-token row
        make_case(B=1, T=150, Hqk=1, Hv=2, Dk=128, dtype="bf16", g_scale=0.3, init_std=0.02,
                  seed=72, name="noalloc_second", g_per_key=True),
    ]
    for x in cases:
        _say(f"noalloc {x.name}: B{x.B} T{x.T} Hv{x.Hv} sequences {x.num_seqs}")
        assert dn.chunk_fwd_path(x.B, x.T, x.Hqk, x.Hv, x.Dk, x.Dv, torch.bfloat16,
                                 num_seqs=x.num_seqs, g_per_key=True) == "channel_gate_two_kernels"
        d = to_inputs(x)
        o1, s1 = _noalloc(x, d)
        o2, s2 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"],
                              cu_seqlens=d["cu"])
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2), "differs from the workspace call"
        o_ref, s_ref = run_oracle(x)
        eo, es = rel_l2(host(o1), o_ref), rel_l2(host(s1), s_ref)
        uo, us, where = per_unit_rel(host(o1), o_ref, host(s1), s_ref, x)
        _say(f"  rel_l2 o={eo:.2e} state={es:.2e}; worst (sequence, head) {uo:.2e} {us:.2e}")
        assert max(eo, es, uo, us) <= tol(x)


def test_noalloc_without_scratch_need():
    """Prompts that need no scratch (one gate per head, the fused kernel at d = 128 and 64)
    run through the allocation-free call unchanged."""
    for D, seed in ((128, 73), (64, 74)):
        x = make_case(B=2, T=200, Hqk=2, Hv=2, Dk=D, dtype="bf16", g_scale=0.1, init_std=0.02,
                      seed=seed, name=f"noalloc_fused_d{D}")
        d = to_inputs(x)
        o1, s1 = _noalloc(x, d)
        o2, s2 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"])
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2)
