"""The reverse pass (dn_recurrent_bwd) on the HIP path against the fp64 reverse-pass
reference oracle/backward.py (needs an MI355X).  The state trace comes from
dn_recurrent_fwd on the same inputs.

Bar: relative L2 over each whole gradient tensor, 1e-4 for fp32 inputs, 1e-2 for bf16.
"""
import sys

import numpy as np
import pytest
import torch

import delta_rule_recurrent_chunked_amd as dn
from oracle.backward import backward as ref_backward
from synth import make_case
from tests.gpu_util import dev_tensor, host, rel_l2, to_inputs, tol

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    "f32_gated_packed_gqa": dict(B=1, Hqk=1, Hv=2, Dk=16, Dv=32, dtype="f32", seqlens=[5, 0, 9, 33],
                                 g_scale=0.2, init_std=0.5, beta_scale=2.0),
    "f32_plain_rows": dict(B=2, T=40, Hqk=2, Dk=32, Dv=16, dtype="f32"),
    "f32_d64_gated": dict(B=1, T=70, Hqk=2, Hv=4, Dk=64, Dv=64, dtype="f32", g_scale=0.1,
                          init_std=0.2),
    "bf16_d128_gated": dict(B=1, T=100, Hqk=2, Hv=2, Dk=128, dtype="bf16", g_scale=0.1,
                            init_std=0.02),
    # a log decay per key channel: dg per (token, head, key channel)
    "f32_channel_gates_packed_gqa": dict(B=1, Hqk=1, Hv=2, Dk=16, Dv=32, dtype="f32",
                                         seqlens=[5, 0, 9, 33], g_scale=0.2, init_std=0.5,
                                         beta_scale=2.0, g_per_key=True),
    "f32_channel_gates_d64": dict(B=1, T=70, Hqk=2, Hv=4, Dk=64, Dv=64, dtype="f32",
                                  g_scale=0.1, init_std=0.2, g_per_key=True),
    "bf16_d128_channel_gates": dict(B=1, T=100, Hqk=2, Hv=2, Dk=128, dtype="bf16",
                                    g_scale=0.1, init_std=0.02, g_per_key=True),
    # raw q and k (N(0,1) draws) normalised inside the rule: dq, dk for the raw inputs
    "f32_in_call_norm_packed_gqa": dict(B=1, Hqk=1, Hv=2, Dk=16, Dv=32, dtype="f32",
                                        seqlens=[5, 0, 9, 33], g_scale=0.2, init_std=0.5,
                                        beta_scale=2.0, qk_raw=True),
    "f32_in_call_norm_channel_gates_d64": dict(B=1, T=70, Hqk=2, Hv=4, Dk=64, Dv=64,
                                               dtype="f32", g_scale=0.1, init_std=0.2,
                                               g_per_key=True, qk_raw=True),
    "bf16_d128_in_call_norm": dict(B=1, T=100, Hqk=2, Hv=2, Dk=128, dtype="bf16", g_scale=0.1,
                                   init_std=0.02, qk_raw=True),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_reverse_pass(name):
    _say(f"reverse pass {name}")
    x = make_case(seed=51, name=name, **CASES[name])
    rng = np.random.default_rng(52)
    N = x.num_seqs
    do = rng.standard_normal((x.B, x.T, x.Hv, x.Dv)).astype(np.float32)
    dfin = rng.standard_normal((N, x.Hv, x.Dk, x.Dv)).astype(np.float32)
    if x.dtype == "bf16":
        from synth import f32_to_bf16_bits
        do_dev = dev_tensor(f32_to_bf16_bits(do))
        do_ref = host(do_dev)
    else:
        do_dev, do_ref = dev_tensor(do), do.astype(np.float64)
    d = to_inputs(x)
    scale = 0.7
    norm = bool(CASES[name].get("qk_raw"))
    _, _, trace = dn.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"],
                                   cu_seqlens=d["cu"], scale=scale, state_trace=True,
                                   qk_l2norm=norm)
    grads = dn.recurrent_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], trace, do_dev,
                             dev_tensor(dfin), cu_seqlens=d["cu"], scale=scale, qk_l2norm=norm)
    torch.cuda.synchronize()
    f = x.f64()
    ref = ref_backward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"], do_ref,
                       dfin.astype(np.float64), x.cu_seqlens, scale, qk_l2norm=norm)
    pairs = [("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dbeta", "dbeta"),
             ("d_initial_state", "dinit")] + ([("dg", "dg")] if x.g is not None else [])
    for got, want in pairs:
        err = rel_l2(host(grads[got]), ref[want])
        _say(f"  {got}: rel_l2 {err:.2e}")
        assert err <= tol(x), got


def test_reverse_pass_graph_replay():
    """dn_recurrent_bwd (reverse kernel, slice sums and, with the in-call normalisation, the
    normalisation's reverse) captured in a HIP graph replays to the eager gradients, every
    replay, with eager work and synchronisations between the replays."""
    _say("reverse pass graph replay")
    x = make_case(B=1, T=90, Hqk=2, Hv=2, Dk=64, Dv=64, dtype="f32", g_scale=0.1, init_std=0.2,
                  seed=54, name="bwd_graph", g_per_key=True, qk_raw=True)
    d = to_inputs(x)
    rng = np.random.default_rng(55)
    do = dev_tensor(rng.standard_normal((1, 90, 2, 64)).astype(np.float32))
    _, _, trace = dn.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"],
                                   state_trace=True, qk_l2norm=True)
    out = {}

    def call():
        out["g"] = dn.recurrent_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], trace,
                                    do, qk_l2norm=True)

    call()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out["g"].items() if v is not None}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    got = out["g"]
    for rep in range(3):
        for v in got.values():
            if v is not None:
                v.zero_()
        torch.ones(1000, device="cuda").sum().item()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(got[k], v), f"replay {rep}: {k} differs from the eager call"


def test_reverse_pass_bitwise_repeatable():
    """Two reverse passes over the same inputs agree bit for bit: every slice share is summed
    in a fixed order (no atomics), with one gate per head and per key channel."""
    _say("reverse pass bitwise repeat")
    for per_key in (False, True):
        x = make_case(B=1, Hqk=1, Hv=2, Dk=128, dtype="bf16", seqlens=[70, 0, 129],
                      g_scale=0.1, init_std=0.02, seed=56, name="bwd_repeat", g_per_key=per_key)
        d = to_inputs(x)
        rng = np.random.default_rng(57)
        from synth import f32_to_bf16_bits
        do = dev_tensor(f32_to_bf16_bits(rng.standard_normal((1, x.T, 2, 128)).astype(np.float32)))
        _, _, trace = dn.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"],
                                       cu_seqlens=d["cu"], state_trace=True)
        runs = [dn.recurrent_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], trace, do,
                                 cu_seqlens=d["cu"]) for _ in range(2)]
        torch.cuda.synchronize()
        for k in runs[0]:
            if runs[0][k] is not None:
                assert torch.equal(runs[0][k], runs[1][k]), (per_key, k)
