"""The token-by-token route (dn_recurrent_fwd) and its per-token state trace against the
fp64 oracle and the explicit-matrix twin (needs an MI355X).

Bar as for every parity test: relative L2 over the whole tensor, 1e-4 for fp32 inputs,
1e-2 for bf16 inputs.
"""
import sys

import numpy as np
import pytest
import torch

import delta_rule_recurrent_chunked_amd as dn
from oracle import brute
from synth import make_case, make_config
from tests.gpu_util import host, rel_l2, to_inputs, tol

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _oracle(x, scale=1.0, qk_l2norm=False):
    import oracle
    f = x.f64()
    return oracle.recurrent(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"],
                            x.cu_seqlens, scale=scale, qk_l2norm=qk_l2norm)


CASES = {
    "config1_f32_d16": (dict(cfg=1), {}),
    "f32_dk32_dv64_gated_init": (dict(B=2, T=77, Hqk=2, Dk=32, Dv=64, dtype="f32", g_scale=0.2,
                                      init_std=0.5, beta_scale=2.0), {}),
    "bf16_d128_packed_gqa": (dict(B=1, Hqk=2, Hv=4, Dk=128, dtype="bf16", seqlens=[70, 0, 1, 129],
                                  g_scale=0.05, init_std=0.02, beta_scale=2.0), {}),
    "bf16_d128_channel_gates": (dict(B=1, T=90, Hqk=1, Hv=2, Dk=128, dtype="bf16", g_scale=0.1,
                                     init_std=0.02, g_per_key=True), {}),
    "bf16_d64_raw_qk": (dict(B=2, T=60, Hqk=2, Dk=64, dtype="bf16", g_scale=0.1, qk_raw=True),
                        dict(qk_l2norm=True)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_recurrent_route(name):
    _say(f"recurrent route {name}")
    spec, kw = CASES[name]
    x = make_config(1) if "cfg" in spec else make_case(seed=41, name=name, **spec)
    d = to_inputs(x)
    o, s, _ = dn.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"],
                               cu_seqlens=d["cu"], scale=0.5, **kw)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x, 0.5, kw.get("qk_l2norm", False))
    eo, es = rel_l2(host(o), o_ref), rel_l2(host(s), s_ref)
    _say(f"  rel_l2 o={eo:.2e} state={es:.2e}")
    assert eo <= tol(x) and es <= tol(x)


def test_state_trace_against_explicit_matrices():
    """The state after every token of packed gated sequences (fp32) against the product form
    with explicit matrices, per sequence from its own initial state; the last trace entry
    of each sequence equals the final state bit for bit."""
    _say("state trace")
    x = make_case(B=1, Hqk=1, Hv=2, Dk=16, Dv=32, dtype="f32", seqlens=[13, 0, 20], g_scale=0.2,
                  init_std=0.5, beta_scale=2.0, seed=42, name="trace")
    d = to_inputs(x)
    o, s, tr = dn.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"],
                                cu_seqlens=d["cu"], state_trace=True)
    torch.cuda.synchronize()
    tr = host(tr)[0]                       # [T, Hv, Dk, Dv]
    f = x.f64()
    cu = x.cu_seqlens
    want = np.zeros_like(tr)
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        for h in range(x.Hv):
            if b == a:
                continue
            Ss = brute.per_token_states(f["k"][0, a:b, 0], f["v"][0, a:b, h], f["beta"][0, a:b, h],
                                        f["g"][0, a:b, h], f["init"][n, h].T)
            want[a:b, h] = np.transpose(Ss, (0, 2, 1))
            assert torch.equal(torch.from_numpy(tr[b - 1, h]), torch.from_numpy(host(s)[n, h]))
    err = rel_l2(tr, want)
    _say(f"  trace rel_l2 {err:.2e}")
    assert err <= 1e-4


def test_recurrent_and_chunked_agree_on_layer_workload():
    """The layer-prefill workload (B4 H16 T2048 d128 bf16) through both routes, each against
    the oracle."""
    _say("recurrent vs chunked, B4 H16 T2048")
    x = make_config(2)
    d = to_inputs(x)
    o1, s1 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], None, None)
    o2, s2, _ = dn.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], None, None)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    for o, s in ((o1, s1), (o2, s2)):
        eo, es = rel_l2(host(o), o_ref), rel_l2(host(s), s_ref)
        _say(f"  rel_l2 o={eo:.2e} state={es:.2e}")
        assert eo <= 1e-2 and es <= 1e-2
