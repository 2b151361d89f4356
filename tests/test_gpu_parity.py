"""HIP path against the fp64 oracle on the same seeded inputs (needs an MI355X).

Bar (relative L2 over the whole tensor, outputs and final states): 1e-4 for fp32
inputs, 1e-2 for bf16 inputs.  Every call goes through the C ABI via the binding.
"""
import sys

import numpy as np
import pytest
import torch

import delta_rule_recurrent_chunked_amd as dn
from synth import make_case, make_config
from tests.gpu_util import host, log_errors, per_unit_rel, rel_l2, run_oracle, to_inputs, tol

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _prefill(x, scale=1.0, chunk=None, **kw):
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"],
                        cu_seqlens=d["cu"], scale=scale,
                        chunk_size=x.chunk if chunk is None else chunk, **kw)
    torch.cuda.synchronize()
    return host(o), host(s)


def _check(x, o, s, scale=1.0, o_ref=None, s_ref=None):
    """The bar on the whole tensors and on every (sequence, value head) separately, so that
    one wrong short sequence or head cannot hide in the aggregate."""
    if o_ref is None:
        o_ref, s_ref = run_oracle(x, scale)
    eo, es = rel_l2(o, o_ref), rel_l2(s, s_ref)
    uo, us, where = per_unit_rel(o, o_ref, s, s_ref, x)
    _say(f"  {x.name}: rel_l2 o={eo:.2e} state={es:.2e}; worst (sequence, head) o={uo:.2e} "
         f"state={us:.2e} at {where} (bar {tol(x):.0e})")
    log_errors(x.name, o=eo, state=es, worst_unit_o=uo, worst_unit_state=us, bar=tol(x),
               worst_unit=where)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert eo <= tol(x) and es <= tol(x)
    assert uo <= tol(x) and us <= tol(x)
    return eo, es


# ------------------------------------------------------------------ the five workloads

@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_prefill_config(cfg):
    _say(f"prefill config {cfg}")
    x = make_config(cfg)
    o, s = _prefill(x)
    _check(x, o, s)


def test_decode_config4():
    _say("decode config 4")
    x = make_config(4)
    d = to_inputs(x)
    state = d["init"].clone()
    o = dn.decode_step(d["q"][:, 0], d["k"][:, 0], d["v"][:, 0], d["beta"][:, 0], d["g"][:, 0],
                       state)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(x)
    _check(x, host(o)[:, None], host(state), o_ref=o_ref, s_ref=s_ref)


# ------------------------------------------------------------------------- edge cases

EDGE = {
    "dk16_dv32_ragged": dict(B=2, T=150, Hqk=2, Dk=16, Dv=32, g_scale=0.1, init_std=0.3),
    "dk32_dv16_gqa": dict(B=1, T=100, Hqk=1, Hv=3, Dk=32, Dv=16, g_scale=0.5, init_std=1.0),
    "dk64_bf16_beta2": dict(B=1, T=200, Hqk=2, Dk=64, dtype="bf16", beta_scale=2.0, g_scale=0.05),
    "short_T_lt_C": dict(B=3, T=7, Hqk=2, Dk=32, dtype="bf16", init_std=0.02),
    "single_token": dict(B=2, T=1, Hqk=2, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02),
    "packed_with_empty": dict(B=1, Hqk=2, Hv=4, Dk=128, dtype="bf16", seqlens=[70, 0, 1, 64, 129, 0],
                              g_scale=0.05, init_std=0.02, beta_scale=2.0),
    "packed_fp32_d16": dict(B=1, Hqk=1, Dk=16, seqlens=[3, 64, 65, 0, 17], g_scale=0.2, init_std=0.5),
    "d128_bf16_ragged_gqa": dict(B=2, T=333, Hqk=2, Hv=4, Dk=128, dtype="bf16", g_scale=0.1,
                                 init_std=0.02),
    "d128_fp32": dict(B=1, T=130, Hqk=2, Dk=128, dtype="f32", g_scale=0.1, init_std=0.02),
    # 70 packed sequences, lengths 0..191
    "many_packed_seqs": dict(B=1, Hqk=2, Hv=2, Dk=128, dtype="bf16",
                             seqlens=[(37 * i) % 192 for i in range(70)], g_scale=0.1,
                             init_std=0.02, beta_scale=2.0),
    # 300 short packed sequences (ordered longest first), lengths 0..40
    "packed_300_seqs": dict(B=1, Hqk=1, Hv=2, Dk=128, dtype="bf16",
                            seqlens=[(29 * i + 3) % 41 for i in range(300)], g_scale=0.1,
                            init_std=0.02, beta_scale=2.0),
    # 600 short packed sequences: more than the kernel ranks longest first (512), so they
    # run in their own order
    "packed_600_seqs_unranked": dict(B=1, Hqk=1, Hv=1, Dk=128, dtype="bf16",
                                     seqlens=[(31 * i + 5) % 37 for i in range(600)], g_scale=0.1,
                                     init_std=0.02),
    # 64 packed sequences, lengths 0..127
    "packed_64_seqs": dict(B=1, Hqk=1, Hv=2, Dk=128, dtype="bf16",
                           seqlens=[(53 * i + 11) % 128 for i in range(64)], g_scale=0.1,
                           init_std=0.02),
    # one long gated sequence: 16 chunks and a 40-token tail, from an initial state
    "d128_bf16_long": dict(B=1, T=1000, Hqk=1, Hv=2, Dk=128, dtype="bf16", g_scale=0.05,
                           init_std=0.02, beta_scale=2.0),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_prefill_edge(name):
    _say(f"prefill edge {name}")
    kw = dict(EDGE[name])
    dtype = kw.pop("dtype", "f32")
    x = make_case(dtype=dtype, seed=7, name=name, **kw)
    o, s = _prefill(x, scale=0.75)
    _check(x, o, s, scale=0.75)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunk_sizes(chunk):
    _say(f"chunk size {chunk}")
    x = make_case(B=1, T=200, Hqk=2, Dk=64, Dv=32, dtype="f32", g_scale=0.1, init_std=0.1,
                  beta_scale=2.0, seed=3, name=f"chunk{chunk}")
    o, s = _prefill(x, chunk=chunk)
    _check(x, o, s)


def test_zero_length_prompt_returns_initial_state():
    _say("T = 0")
    x = make_case(B=2, T=0, Hqk=2, Dk=16, dtype="f32", init_std=1.0, seed=1)
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], None, d["init"])
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.equal(s, d["init"])


def test_gqa_equals_explicit_repeat():
    _say("GQA vs repeated heads")
    x = make_case(B=1, T=190, Hqk=2, Hv=6, Dk=128, dtype="bf16", g_scale=0.1, seed=4)
    d = to_inputs(x)
    o1, s1 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"])
    qr = d["q"].repeat_interleave(3, dim=2).contiguous()
    kr = d["k"].repeat_interleave(3, dim=2).contiguous()
    o2, s2 = dn.chunk_fwd(qr, kr, d["v"], d["beta"], d["g"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_final_state_may_alias_initial_state():
    _say("aliasing")
    x = make_case(B=2, T=97, Hqk=2, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02, seed=5)
    d = to_inputs(x)
    o1, s1 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"])
    st = d["init"].clone()
    o2, s2 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], st, final_state=st)
    torch.cuda.synchronize()
    assert s2.data_ptr() == st.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(s1, st)


def test_split_continuation():
    """prefill(0..T) == prefill(t0..T) started from prefill(0..t0)'s final state."""
    _say("split continuation")
    x = make_case(B=1, T=300, Hqk=2, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02, seed=6,
                  name="split_continuation")
    d = to_inputs(x)
    t0 = 137
    oa, sa = dn.chunk_fwd(d["q"][:, :t0].contiguous(), d["k"][:, :t0].contiguous(),
                          d["v"][:, :t0].contiguous(), d["beta"][:, :t0].contiguous(),
                          d["g"][:, :t0].contiguous(), d["init"])
    ob, sb = dn.chunk_fwd(d["q"][:, t0:].contiguous(), d["k"][:, t0:].contiguous(),
                          d["v"][:, t0:].contiguous(), d["beta"][:, t0:].contiguous(),
                          d["g"][:, t0:].contiguous(), sa)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(x)
    o = np.concatenate([host(oa), host(ob)], axis=1)
    _check(x, o, host(sb), o_ref=o_ref, s_ref=s_ref)


def test_prefill_equals_decode_steps():
    """T decode steps from the same start reach the oracle's result as well."""
    _say("decode steps vs oracle")
    x = make_case(B=3, T=40, Hqk=2, Hv=4, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02,
                  beta_scale=2.0, seed=8, name="prefill_vs_decode_steps")
    d = to_inputs(x)
    state = d["init"].clone()
    outs = []
    for t in range(x.T):
        outs.append(dn.decode_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                   d["v"][:, t].contiguous(), d["beta"][:, t].contiguous(),
                                   d["g"][:, t].contiguous(), state))
    torch.cuda.synchronize()
    o = np.stack([host(t) for t in outs], axis=1)
    _check(x, o, host(state))


@pytest.mark.parametrize("Dk,Dv,dtype", [(16, 16, "f32"), (32, 64, "bf16"), (64, 128, "f32"),
                                         (128, 16, "bf16"), (128, 128, "f32")])
def test_decode_shapes(Dk, Dv, dtype):
    _say(f"decode {Dk}x{Dv} {dtype}")
    x = make_case(B=5, T=1, Hqk=2, Hv=4, Dk=Dk, Dv=Dv, dtype=dtype, g_scale=0.1, init_std=0.5,
                  seed=9, decode=True, name=f"decode{Dk}x{Dv}{dtype}")
    d = to_inputs(x)
    state = d["init"].clone()
    o = dn.decode_step(d["q"][:, 0], d["k"][:, 0], d["v"][:, 0], d["beta"][:, 0], d["g"][:, 0],
                       state, scale=0.5)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(x, 0.5)
    _check(x, host(o)[:, None], host(state), o_ref=o_ref, s_ref=s_ref)


def test_outputs_fully_written_and_deterministic():
    """Outputs poisoned with NaN are overwritten everywhere; two runs agree bit for bit."""
    _say("poison + determinism")
    x = make_case(B=1, Hqk=2, Hv=4, Dk=128, dtype="bf16", seqlens=[100, 1, 0, 333],
                  g_scale=0.1, init_std=0.02, seed=10)
    d = to_inputs(x)
    outs = []
    for _ in range(2):
        o = torch.full((1, x.T, 4, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        s = torch.full((4, 4, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
        dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], cu_seqlens=d["cu"],
                     out=o, final_state=s)
        torch.cuda.synchronize()
        assert not torch.isnan(o).any() and not torch.isnan(s).any()
        outs.append((o, s))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_graph_replay_matches_eager():
    """A HIP graph capturing prefill and decode calls replays to the eager results, every
    replay, with eager work and synchronisations between replays (the library allocates
    nothing and records no memset inside a call)."""
    _say("graph replay")
    x = make_config(2)
    d = to_inputs(x)
    B, T, H, D = x.B, x.T, x.Hv, x.Dk
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    fs = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    y = make_config(4)
    e = to_inputs(y)
    st = e["init"].clone()
    od = torch.empty((y.B, y.Hv, y.Dv), dtype=torch.bfloat16, device="cuda")
    dargs = (e["q"][:, 0].contiguous(), e["k"][:, 0].contiguous(), e["v"][:, 0].contiguous(),
             e["beta"][:, 0].contiguous(), e["g"][:, 0].contiguous())

    def calls():
        dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], None, None, out=o, final_state=fs)
        dn.decode_step(*dargs, st, out=od)

    st.copy_(e["init"])
    calls()
    torch.cuda.synchronize()
    ref = (o.clone(), fs.clone(), od.clone(), st.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        st.copy_(e["init"])
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        o.zero_(), fs.zero_(), od.zero_()
        st.copy_(e["init"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((o, fs, od, st), ref, ("o", "final_state", "decode o", "state")):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager call"
        _ = (o.float().sum() + 1).item()   # eager work between replays


def test_decode_ungated_workload():
    """The decode workload without a gate (the plain rule: 256 sequences x 32 heads, d128 bf16,
    state in place)."""
    _say("decode 256 x 32, no gate")
    x = make_case(B=256, T=1, Hqk=32, Dk=128, dtype="bf16", init_std=0.02, seed=0, decode=True,
                  name="decode_plain")
    d = to_inputs(x)
    state = d["init"].clone()
    o = dn.decode_step(d["q"][:, 0], d["k"][:, 0], d["v"][:, 0], d["beta"][:, 0], None, state)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(x)
    _check(x, host(o)[:, None], host(state), o_ref=o_ref, s_ref=s_ref)

