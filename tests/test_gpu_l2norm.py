"""In-rule q/k L2 normalisation (DN_QK_L2NORM) on the HIP path against the fp64 oracle
(needs an MI355X).

The caller hands raw q and k (N(0, 1) draws, as a projection would give them); the call
replaces each by x / sqrt(|x|^2 + eps) before the rule.  The oracle normalises in fp64
from the same bf16/fp32 bits.  Bar as for every parity test: relative L2 over the whole
tensor, 1e-4 for fp32 inputs, 1e-2 for bf16 inputs, outputs and final states.
"""
import sys

import numpy as np
import pytest
import torch

import delta_rule_recurrent_chunked_amd as dn
from synth import make_case
from tests.gpu_util import host, rel_l2, to_inputs, tol

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _oracle(x, scale=1.0, eps=1e-6):
    import oracle
    f = x.f64()
    return oracle.recurrent(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"],
                            x.cu_seqlens, scale=scale, qk_l2norm=True, eps=eps)


def _check(x, o, s, o_ref, s_ref):
    eo, es = rel_l2(o, o_ref), rel_l2(s, s_ref)
    _say(f"  {x.name}: rel_l2 o={eo:.2e} state={es:.2e} (bar {tol(x):.0e})")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert eo <= tol(x) and es <= tol(x)


CASES = {
    # the matrix-core path (bf16, d = 128): plain and gated, ragged, GQA, packed, long
    "fused_plain_ragged": dict(B=2, T=333, Hqk=2, Dk=128, dtype="bf16"),
    "fused_gated_packed_gqa": dict(B=1, Hqk=2, Hv=4, Dk=128, dtype="bf16",
                                   seqlens=[70, 0, 1, 64, 129, 0], g_scale=0.05,
                                   init_std=0.02, beta_scale=2.0),
    "fused_gated_long": dict(B=1, T=1000, Hqk=1, Hv=2, Dk=128, dtype="bf16", g_scale=0.05,
                             init_std=0.02, beta_scale=2.0),
    # the same kernel at d = 64
    "fused_d64_plain_ragged": dict(B=2, T=333, Hqk=2, Dk=64, dtype="bf16"),
    "fused_d64_gated_packed_gqa": dict(B=1, Hqk=2, Hv=4, Dk=64, dtype="bf16",
                                       seqlens=[70, 0, 1, 64, 129, 0], g_scale=0.05,
                                       init_std=0.02, beta_scale=2.0),
    # the vector-ALU path: fp32 (1e-4 bar) and bf16 at other head sizes
    "generic_f32_d64": dict(B=1, T=150, Hqk=2, Dk=64, dtype="f32", g_scale=0.1, init_std=0.3),
    "generic_f32_d128_packed": dict(B=1, Hqk=1, Hv=2, Dk=128, dtype="f32",
                                    seqlens=[3, 64, 65, 0, 17], g_scale=0.2, init_std=0.02),
    "generic_bf16_d32_dv16": dict(B=2, T=100, Hqk=2, Dk=32, Dv=16, dtype="bf16", g_scale=0.1),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_l2norm(name):
    _say(f"l2norm prefill {name}")
    kw = dict(CASES[name])
    x = make_case(seed=11, name=name, qk_raw=True, **kw)
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"],
                        cu_seqlens=d["cu"], scale=0.75, qk_l2norm=True, l2norm_eps=1e-6)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x, 0.75)
    _check(x, host(o), host(s), o_ref, s_ref)


def test_prefill_l2norm_eps_zero():
    """eps = 0 (a pure normalisation) on the matrix-core path, gated, with an initial state."""
    _say("l2norm prefill eps = 0")
    x = make_case(B=1, T=200, Hqk=2, Hv=2, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02,
                  seed=12, name="eps0", qk_raw=True)
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"],
                        qk_l2norm=True, l2norm_eps=0.0)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x, eps=0.0)
    _check(x, host(o), host(s), o_ref, s_ref)


def test_prefill_l2norm_layer_workload():
    """The layer-prefill workload (B4 H16 T2048 d128 bf16, no decay) handed raw q and k."""
    _say("l2norm prefill B4 H16 T2048")
    x = make_case(B=4, T=2048, Hqk=16, Dk=128, dtype="bf16", seed=0, name="layer_raw_qk",
                  qk_raw=True)
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], None, None, qk_l2norm=True)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    _check(x, host(o), host(s), o_ref, s_ref)


def test_prefill_l2norm_of_unit_inputs_matches_plain_call():
    """Inputs already of unit norm: normalising inside the call changes only rounding."""
    _say("l2norm of unit vectors vs plain call")
    x = make_case(B=1, T=300, Hqk=2, Hv=4, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02,
                  seed=13, name="unit")
    d = to_inputs(x)
    o1, s1 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"])
    o2, s2 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], qk_l2norm=True)
    torch.cuda.synchronize()
    assert rel_l2(host(o2), host(o1)) < 5e-3 and rel_l2(host(s2), host(s1)) < 5e-3


@pytest.mark.parametrize("Dk,Dv,dtype", [(128, 128, "bf16"), (64, 32, "f32"), (16, 16, "f32")])
def test_decode_l2norm(Dk, Dv, dtype):
    _say(f"l2norm decode {Dk}x{Dv} {dtype}")
    x = make_case(B=6, T=1, Hqk=2, Hv=4, Dk=Dk, Dv=Dv, dtype=dtype, g_scale=0.1, init_std=0.5,
                  seed=14, decode=True, name=f"decode{Dk}x{Dv}{dtype}", qk_raw=True)
    d = to_inputs(x)
    state = d["init"].clone()
    o = dn.decode_step(d["q"][:, 0], d["k"][:, 0], d["v"][:, 0], d["beta"][:, 0], d["g"][:, 0],
                       state, scale=0.5, qk_l2norm=True)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x, 0.5)
    _check(x, host(o)[:, None], host(state), o_ref, s_ref)


def test_l2norm_prefill_equals_decode_steps():
    """T decode steps from the zero state equal one normalising prefill call."""
    _say("l2norm prefill vs decode steps")
    x = make_case(B=2, T=40, Hqk=2, Hv=2, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02,
                  seed=15, name="steps", qk_raw=True)
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], qk_l2norm=True)
    state = d["init"].clone()
    outs = []
    for t in range(x.T):
        outs.append(dn.decode_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                   d["v"][:, t].contiguous(), d["beta"][:, t].contiguous(),
                                   d["g"][:, t].contiguous(), state, qk_l2norm=True))
    torch.cuda.synchronize()
    od = np.stack([host(t) for t in outs], axis=1)
    o_ref, s_ref = _oracle(x)
    _check(x, od, host(state), o_ref, s_ref)
    _check(x, host(o), host(s), o_ref, s_ref)


def test_prefill_l2norm_gated_gqa_workload():
    """The gated GQA workload (B2, 16 q/k heads -> 32 v heads, T8192, d128 bf16) handed raw
    q and k: the gated matrix-core path with the normalisation folded in."""
    _say("l2norm prefill gated GQA B2 T8192")
    x = make_case(B=2, T=8192, Hqk=16, Hv=32, Dk=128, dtype="bf16", g_scale=0.1, seed=0,
                  name="gated_gqa_raw_qk", qk_raw=True)
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], None, qk_l2norm=True)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    _check(x, host(o), host(s), o_ref, s_ref)


def test_l2norm_graph_replay_matches_eager():
    """A HIP graph of a normalising prefill and decode replays to the eager results."""
    _say("l2norm graph replay")
    x = make_case(B=2, T=300, Hqk=2, Hv=4, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02,
                  seed=16, name="graph", qk_raw=True)
    d = to_inputs(x)
    o = torch.empty((x.B, x.T, x.Hv, x.Dv), dtype=torch.bfloat16, device="cuda")
    fs = torch.empty((x.B, x.Hv, x.Dk, x.Dv), dtype=torch.float32, device="cuda")
    st = d["init"].clone()
    od = torch.empty((x.B, x.Hv, x.Dv), dtype=torch.bfloat16, device="cuda")
    dargs = tuple(t[:, 0].contiguous() for t in (d["q"], d["k"], d["v"], d["beta"], d["g"]))

    def calls():
        dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], out=o, final_state=fs,
                     qk_l2norm=True)
        dn.decode_step(*dargs, st, out=od, qk_l2norm=True)

    calls()
    torch.cuda.synchronize()
    ref = (o.clone(), fs.clone(), od.clone(), st.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        st.copy_(d["init"])
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        o.zero_(), fs.zero_(), od.zero_()
        st.copy_(d["init"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((o, fs, od, st), ref, ("o", "final_state", "decode o", "state")):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager call"
