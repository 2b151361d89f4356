"""The readout epilogue (normalisation over d_v, silu output gate) on the HIP path against
the fp64 reference oracle/epilogue.py (needs an MI355X): standalone over a prefill's
output (dn_norm_gate) and fused into the decode step (dn_decode_step_ex).

Bar: relative L2 over the whole tensor, 1e-4 for fp32, 1e-2 for bf16.
"""
import sys

import numpy as np
import pytest
import torch

import delta_rule_recurrent_chunked_amd as dn
from oracle.epilogue import norm_gate as ref_norm_gate
from synth import make_case, make_epilogue_inputs, to_f64
from tests.gpu_util import dev_tensor, host, rel_l2, run_oracle, to_inputs

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bar(dtype):
    return 1e-4 if dtype == "f32" else 1e-2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Dv", [16, 32, 64, 128])
@pytest.mark.parametrize("kind", ["rms", "layer"])
def test_norm_gate_standalone(dtype, Dv, kind):
    _say(f"norm_gate {kind} Dv={Dv} {dtype}")
    shape = (2, 37, 3, Dv)          # 222 rows: not a multiple of the rows per workgroup
    e = make_epilogue_inputs(shape, dtype, seed=Dv)
    o, gate = dev_tensor(e["o"]), dev_tensor(e["gate"])
    w, b = dev_tensor(e["weight"]), dev_tensor(e["bias"]) if kind == "layer" else None
    y = dn.norm_gate(o, kind, 1e-5, w, b, gate)
    torch.cuda.synchronize()
    want = ref_norm_gate(to_f64(e["o"]), kind, 1e-5, e["weight"], None if b is None else e["bias"],
                         to_f64(e["gate"]))
    err = rel_l2(host(y), want)
    _say(f"  rel_l2 {err:.2e}")
    assert err <= _bar(dtype)


def test_norm_gate_in_place_without_gate_or_weight():
    _say("norm_gate in place, no gate, no weight")
    e = make_epilogue_inputs((1, 50, 4, 128), "bf16", seed=5)
    o = dev_tensor(e["o"])
    y = dn.norm_gate(o, "layer", 1e-6, out=o)
    torch.cuda.synchronize()
    assert y.data_ptr() == o.data_ptr()
    want = ref_norm_gate(to_f64(e["o"]), "layer", 1e-6)
    assert rel_l2(host(o), want) <= 1e-2


def test_prefill_then_norm_gate_layer_workload():
    """The layer-prefill workload (B4 H16 T2048 d128 bf16) followed by the epilogue, against
    the oracle's fp64 readout put through the reference epilogue."""
    _say("prefill + norm_gate, B4 H16 T2048")
    x = make_case(B=4, T=2048, Hqk=16, Dk=128, dtype="bf16", seed=0, name="layer")
    e = make_epilogue_inputs((4, 2048, 16, 128), "bf16", seed=1)
    d = to_inputs(x)
    o, _ = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], None, None, output_final_state=False)
    y = dn.norm_gate(o, "rms", 1e-6, dev_tensor(e["weight"]), None, dev_tensor(e["gate"]))
    torch.cuda.synchronize()
    o_ref, _ = run_oracle(x)
    want = ref_norm_gate(o_ref, "rms", 1e-6, e["weight"], None, to_f64(e["gate"]))
    err = rel_l2(host(y), want)
    _say(f"  rel_l2 {err:.2e}")
    assert err <= 1e-2


@pytest.mark.parametrize("Dk,Dv,dtype,kind", [(128, 128, "bf16", "rms"), (128, 128, "bf16", "layer"),
                                              (64, 32, "f32", "layer"), (16, 16, "f32", "rms"),
                                              (32, 64, "f32", "rms")])
def test_decode_fused_epilogue(Dk, Dv, dtype, kind):
    _say(f"decode + fused epilogue {Dk}x{Dv} {dtype} {kind}")
    x = make_case(B=7, T=1, Hqk=2, Hv=4, Dk=Dk, Dv=Dv, dtype=dtype, g_scale=0.1, init_std=0.5,
                  seed=31, decode=True, name="dec_ep")
    e = make_epilogue_inputs((7, 4, Dv), dtype, seed=32)
    d = to_inputs(x)
    state = d["init"].clone()
    b = dev_tensor(e["bias"]) if kind == "layer" else None
    y = dn.decode_step(d["q"][:, 0], d["k"][:, 0], d["v"][:, 0], d["beta"][:, 0], d["g"][:, 0],
                       state, scale=0.5, norm=kind, norm_eps=1e-5, norm_weight=dev_tensor(e["weight"]),
                       norm_bias=b, out_gate=dev_tensor(e["gate"]))
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(x, 0.5)
    want = ref_norm_gate(o_ref[:, 0], kind, 1e-5, e["weight"], None if b is None else e["bias"],
                         to_f64(e["gate"]))
    ey, es = rel_l2(host(y), want), rel_l2(host(state), s_ref)
    _say(f"  rel_l2 y={ey:.2e} state={es:.2e}")
    assert ey <= _bar(dtype) and es <= _bar(dtype)


def test_decode_fused_epilogue_workload():
    """The decode workload (256 sequences x 32 heads, d128 bf16, gated, state in place) with
    the RMS epilogue and output gate fused."""
    _say("decode 256 x 32 + fused epilogue")
    x = make_case(B=256, T=1, Hqk=32, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02, seed=0,
                  decode=True, name="dec_ep_full")
    e = make_epilogue_inputs((256, 32, 128), "bf16", seed=2)
    d = to_inputs(x)
    state = d["init"].clone()
    y = dn.decode_step(d["q"][:, 0], d["k"][:, 0], d["v"][:, 0], d["beta"][:, 0], d["g"][:, 0],
                       state, norm="rms", norm_weight=dev_tensor(e["weight"]),
                       out_gate=dev_tensor(e["gate"]))
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(x)
    want = ref_norm_gate(o_ref[:, 0], "rms", 1e-6, e["weight"], None, to_f64(e["gate"]))
    assert rel_l2(host(y), want) <= 1e-2 and rel_l2(host(state), s_ref) <= 1e-2


def test_graph_replay_of_epilogue_and_recurrent_calls():
    """A HIP graph holding dn_norm_gate, a decode step with the fused epilogue and the
    token-by-token route (with its trace) replays to the eager results, every replay."""
    _say("graph replay: epilogue, fused decode, recurrent route")
    x = make_case(B=2, T=100, Hqk=2, Hv=4, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02,
                  seed=33, name="graph")
    e = make_epilogue_inputs((2, 100, 4, 128), "bf16", seed=34)
    d = to_inputs(x)
    w, gate = dev_tensor(e["weight"]), dev_tensor(e["gate"])
    o = torch.empty((2, 100, 4, 128), dtype=torch.bfloat16, device="cuda")
    fs = torch.empty((2, 4, 128, 128), dtype=torch.float32, device="cuda")
    y = torch.empty_like(o)
    st = d["init"].clone()
    od = torch.empty((2, 4, 128), dtype=torch.bfloat16, device="cuda")
    dargs = tuple(t[:, 0].contiguous() for t in (d["q"], d["k"], d["v"], d["beta"], d["g"]))
    dgate = gate[:, 0].contiguous()
    trace = {}

    def calls():
        _, _, tr = dn.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], out=o,
                                    final_state=fs, state_trace=True)
        trace["t"] = tr
        dn.norm_gate(o, "layer", 1e-5, w, None, gate, out=y)
        dn.decode_step(*dargs, st, out=od, norm="rms", norm_weight=w, out_gate=dgate)

    calls()
    torch.cuda.synchronize()
    ref = (o.clone(), fs.clone(), y.clone(), od.clone(), st.clone(), trace["t"].clone())
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
    tr = trace["t"]
    for rep in range(3):
        o.zero_(), fs.zero_(), y.zero_(), od.zero_(), tr.zero_()
        st.copy_(d["init"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((o, fs, y, od, st, tr), ref,
                                   ("o", "final_state", "y", "decode y", "state", "trace")):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager call"
