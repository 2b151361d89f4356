"""The bf16 d = 64 prompt on the matrix cores (the one-launch kernel at d_k = d_v = 64)
against the fp64 oracle, through the C ABI (needs an MI355X).

Bar: relative L2 1e-2 (bf16 inputs) over whole tensors and per (sequence, value head).
The cases cover ragged tails, packed batches with empty and one-token sequences, initial
states, GQA with the (sequence, q/k head) count a multiple of 8 (the XCD-grouped workgroup
order) and not, no gate, strong decay, write strengths up to 2, a long sequence, graph
replay, and a final state that aliases the initial one.
"""
import sys

import numpy as np
import pytest
import torch

import delta_rule_recurrent_chunked_amd as dn
from synth import make_case
from tests.gpu_util import host, log_errors, per_unit_rel, rel_l2, run_oracle, to_inputs, tol

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    "d64_plain_ragged": dict(B=2, T=333, Hqk=2, init_std=0.3),
    "d64_gated_gqa_xcd": dict(B=2, T=300, Hqk=4, Hv=8, g_scale=0.1, init_std=0.02, beta_scale=2.0),
    "d64_gqa_3_to_6": dict(B=1, T=200, Hqk=3, Hv=6, g_scale=0.1, init_std=0.1),
    "d64_packed_empty": dict(B=1, Hqk=2, Hv=4, seqlens=[70, 0, 1, 64, 129, 0, 200], g_scale=0.05,
                             init_std=0.02, beta_scale=2.0),
    "d64_strong_decay": dict(B=2, T=257, Hqk=2, g_scale=3.0, init_std=1.0),
    "d64_long": dict(B=1, T=2000, Hqk=1, Hv=2, g_scale=0.05, init_std=0.02, beta_scale=2.0),
    "d64_short": dict(B=3, T=7, Hqk=2, g_scale=0.1),
    "d64_many_packed": dict(B=1, Hqk=2, Hv=2, seqlens=[(37 * i) % 150 for i in range(40)],
                            g_scale=0.1, init_std=0.02),
    # more packed sequences than the kernel ranks longest first (512)
    "d64_packed_600_unranked": dict(B=1, Hqk=1, Hv=1, seqlens=[(31 * i + 5) % 37 for i in range(600)],
                                    g_scale=0.1, init_std=0.02),
}


def _run(x, scale, workspace=None):
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], cu_seqlens=d["cu"],
                        scale=scale, workspace=workspace)
    torch.cuda.synchronize()
    return host(o), host(s)


def _check(x, o, s, scale):
    o_ref, s_ref = run_oracle(x, scale)
    eo, es = rel_l2(o, o_ref), rel_l2(s, s_ref)
    uo, us, where = per_unit_rel(o, o_ref, s, s_ref, x)
    _say(f"  {x.name}: rel_l2 o={eo:.2e} state={es:.2e}; worst (sequence, head) o={uo:.2e} "
         f"state={us:.2e} at {where}")
    log_errors(x.name, o=eo, state=es, worst_unit_o=uo, worst_unit_state=us, bar=tol(x),
               worst_unit=where)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert max(eo, es, uo, us) <= tol(x)


@pytest.mark.parametrize("name", sorted(CASES))
def test_d64_prompt(name):
    x = make_case(Dk=64, dtype="bf16", seed=17, name=name, **CASES[name])
    _say(f"d64 prompt {name}: B{x.B} T{x.T} {x.Hqk}->{x.Hv} heads, {x.num_seqs} sequences")
    assert dn.chunk_fwd_path(x.B, x.T, x.Hqk, x.Hv, 64, 64, torch.bfloat16,
                             num_seqs=x.num_seqs) == "fused"
    o, s = _run(x, 0.8)
    _check(x, o, s, 0.8)


def test_d64_needs_no_workspace_and_other_forms_stay_on_the_vector_kernel():
    assert dn.workspace_bytes(1, 128, 2, 2, 64, 64, torch.bfloat16) == 0
    assert dn.chunk_fwd_path(1, 128, 2, 2, 64, 64, torch.bfloat16, workspace_bytes=0) == "fused"
    assert dn.chunk_fwd_path(1, 128, 2, 2, 64, 64, torch.bfloat16, qk_l2norm=True) == "fused"
    assert dn.chunk_fwd_path(1, 128, 2, 2, 64, 64, torch.float32) == "vector"
    assert dn.chunk_fwd_path(1, 128, 2, 2, 64, 64, torch.bfloat16, chunk_size=32) == "vector"
    assert dn.chunk_fwd_path(1, 128, 2, 2, 64, 32, torch.bfloat16) == "vector"


def test_d64_graph_replay():
    """A HIP graph of the launch replays to the eager result, every replay."""
    x = make_case(B=2, T=500, Hqk=2, Hv=4, Dk=64, dtype="bf16", g_scale=0.1, init_std=0.02,
                  seed=9, name="d64_graph")
    d = to_inputs(x)
    o = torch.empty((x.B, x.T, x.Hv, 64), dtype=torch.bfloat16, device="cuda")
    fs = torch.empty((x.B, x.Hv, 64, 64), dtype=torch.float32, device="cuda")

    def call():
        dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], out=o, final_state=fs)

    call()
    torch.cuda.synchronize()
    ref = (o.clone(), fs.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        o.zero_(), fs.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(fs, ref[1]), f"replay {rep} differs"
        _ = (o.float().sum() + 1).item()


def test_d64_final_state_may_alias_initial_state():
    """Each chain wave reads its columns of the initial state before it writes the final
    state, so one tensor can serve as both (the state updated in place)."""
    x = make_case(B=2, T=200, Hqk=2, Dk=64, dtype="bf16", g_scale=0.1, init_std=0.1, seed=11,
                  name="d64_alias")
    d = to_inputs(x)
    o1, s1 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"])
    st = d["init"].clone()
    o2, s2 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], st, final_state=st)
    torch.cuda.synchronize()
    assert s2.data_ptr() == st.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(s1, st)


def test_d64_zero_length_prompt_returns_initial_state():
    x = make_case(B=2, T=0, Hqk=2, Dk=64, dtype="bf16", init_std=1.0, seed=12, name="d64_T0")
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], None, d["init"])
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(s, d["init"])
